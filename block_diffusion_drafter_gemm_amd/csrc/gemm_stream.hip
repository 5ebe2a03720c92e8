// Persistent weight-streaming GEMM for up to 16 activation rows: the batch-1
// (and small-batch) projections of the drafter step, bound by HBM bandwidth.
//
// out[M, N] = A[M, K] * W[N, K]^T with M <= 16, W row-major [out, in].
//
// One 16-wave workgroup runs per compute unit and walks 16-column tiles
// round-robin (tile = block, block + grid, ...).  For every tile the 16 waves
// split the k-chunks (32 wide) evenly and their partial tiles are summed
// through LDS in wave order; the next tile's weight fragments are already in
// flight while a tile is reduced and its epilogue runs, so the HBM stream does
// not stop between tiles.
//
// The activation rows are staged in LDS once per workgroup when all of K fits
// (K <= 4096 in bf16): as a copy, or as RMSNorm(X) * gain computed from the fp32
// residual stream (optionally gathered from the embedding first).  Longer K
// (the down projection, the context-fusion projection) reads the activation
// fragments straight from global memory, prefetched with the weights.
//
// Column maps and epilogues are those of the few-rows GEMM (RoPE pairs, SwiGLU
// pairs, residual add, storage, per-row argmax).
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kSWaves = 16;
constexpr int kSThreads = kSWaves * 64;
constexpr int kSResBytes = 128 * 1024;   // LDS budget of the resident activation rows

enum AMode { A_GLOBAL = 0, A_COPY = 1, A_NORM = 2, A_EMBED_NORM = 3 };

template <typename T>
__host__ __device__ constexpr int stream_res_k() {
  return kSResBytes / (16 * (int)sizeof(T));
}

template <int EPI>
__device__ __forceinline__ int s_weight_row(const GemmArgs &a, int t, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    return c < 8 ? t * 8 + c : a.ffn + t * 8 + (c - 8);
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int tph = a.hd / 16;
    const int h = t / tph, j0 = (t - h * tph) * 8;
    return h * a.hd + (c < 8 ? j0 + c : a.hd / 2 + j0 + (c - 8));
  } else {
    return t * 16 + c;
  }
}

// Epilogue of one 16 x 16 tile held in LDS (ct, row-major [16][16]).
template <typename T, int EPI>
__device__ __forceinline__ void s_epilogue(const GemmArgs &a, const float *ct, int t, int layer, float *best_v,
                                           int *best_i, const double *inv_freq) {
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    if (tid < 256) {
      const int r = tid >> 4, c = tid & 15;
      if (r < a.M) {
        const int n = t * 16 + c;
        const float v = ct[tid];
        if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)r * a.ldo + n, v);
        else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)r * a.ldo + n] = v;
        else a.X[(size_t)r * a.ldx + n] += v;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (tid < 128) {
      const int r = tid >> 3, c = tid & 7;
      if (r < a.M) {
        const float gt = ct[r * 16 + c], up = ct[r * 16 + 8 + c];
        Storage<T>::store((T *)a.out, (size_t)r * a.ldo + t * 8 + c, gt / (1.0f + expf(-gt)) * up);
      }
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    if (tid < 128) {
      const int r = tid >> 3, c = tid & 7;
      if (r < a.M) {
        const int hd = a.hd, half = hd / 2;
        const int qcols = (EPI == EPI_QKV) ? a.nq * hd : 0;
        const int kcols = a.nkv * hd;
        const int j0 = (t % (hd / 16)) * 8;
        const int n = s_weight_row<EPI>(a, t, c);
        const float x1 = ct[r * 16 + c], x2 = ct[r * 16 + 8 + c];
        int pos;
        size_t slot = 0;
        if constexpr (EPI == EPI_QKV) {
          const int s = r / a.block_size, j = r - s * a.block_size;
          pos = a.ctx_len[s] + j;
        } else {
          pos = a.pos[r];
          const int s = a.seq[r];
          const int page = a.block_table[(size_t)s * a.max_pages + pos / a.page_size];
          slot = (size_t)layer * a.cache_layer_stride + ((size_t)page * a.page_size + (pos % a.page_size)) * kcols;
        }
        float lo = x1, hi = x2;
        if (n < qcols + kcols) {
          float cs, sn;
          rope_cs_inv(pos, inv_freq[j0 + c], &cs, &sn);
          lo = x1 * cs - x2 * sn;
          hi = x2 * cs + x1 * sn;
        }
        T *dst;
        size_t off;
        if (n < qcols) {
          dst = (T *)a.q_out;
          off = (size_t)r * qcols + n;
        } else if (n < qcols + kcols) {
          dst = (T *)a.k_out;
          off = (EPI == EPI_QKV ? (size_t)r * kcols : slot) + (n - qcols);
        } else {
          dst = (T *)a.v_out;
          off = (EPI == EPI_QKV ? (size_t)r * kcols : slot) + (n - qcols - kcols);
        }
        Storage<T>::store(dst, off, lo);
        Storage<T>::store(dst, off + half, hi);
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // running (max, lowest id) per row across this workgroup's tiles; tiles
    // arrive in increasing order, so a strict comparison keeps the lowest id
    if (tid < 16) {
      float b = ct[tid * 16];
      int bc = 0;
#pragma unroll
      for (int c = 1; c < 16; ++c) {
        const float v = ct[tid * 16 + c];
        if (v > b) { b = v; bc = c; }
      }
      if (b > *best_v) { *best_v = b; *best_i = t * 16 + bc; }
    }
  }
}

// One batch of U k-chunks: weight fragments (and, when the activations are not
// resident, activation fragments) for one lane.
template <typename T, int U, bool RES>
struct StreamBuf {
  Frag<T> w[U];
  Frag<T> x[RES ? 1 : U];

  template <int EPI>
  __device__ __forceinline__ void issue(const GemmArgs &a, const T *W, const T *arow, bool row_ok, int t, int c0,
                                        int cend) {
    const int ln = threadIdx.x & 15, g = (threadIdx.x >> 4) & 3;
    const T *wp = W + (size_t)s_weight_row<EPI>(a, t, ln) * a.ldw + 8 * g;
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (c0 + j < cend) w[j].load(wp + 32 * (c0 + j)); else w[j].zero();
      if constexpr (!RES) {
        if (c0 + j < cend && row_ok) x[j].load(arow + 32 * (c0 + j)); else x[j].zero();
      }
    }
  }

  __device__ __forceinline__ f32x4 compute(f32x4 acc, const T *arow, int c0, int cend) const {
#pragma unroll
    for (int j = 0; j < U; ++j) {
      if (c0 + j < cend) {
        if constexpr (RES) {
          Frag<T> af;
          af.load(arow + 32 * (c0 + j));
          acc = mma(acc, af, w[j]);
        } else {
          acc = mma(acc, x[j], w[j]);
        }
      }
    }
    return acc;
  }
};

// Tile finished: sum the 16 waves' partial tiles in wave order, run the epilogue.
template <typename T, int EPI>
__device__ __forceinline__ void s_finish_tile(const GemmArgs &a, f32x4 &acc, float (*red)[256], float *ct, int t,
                                              int layer, float *best_v, int *best_i, const double *inv_freq) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
#pragma unroll
  for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + ln] = f4get(acc, i);
  acc = f32x4{0.f, 0.f, 0.f, 0.f};
  lds_barrier();
  if (tid < 256) {
    float sm = 0.f;
#pragma unroll
    for (int w = 0; w < kSWaves; ++w) sm += red[w][tid];
    ct[tid] = sm;
  }
  lds_barrier();
  s_epilogue<T, EPI>(a, ct, t, layer, best_v, best_i, inv_freq);
}

template <typename T, int EPI, int AM>
__global__ __launch_bounds__(kSThreads) void gemm_stream_kernel(const GemmArgs a) {
  constexpr bool RES = AM != A_GLOBAL;
  constexpr int KR = stream_res_k<T>();                        // resident k capacity
  constexpr int ASTR = (RES ? KR : 0) * (int)sizeof(T) + 16;   // bytes per resident row
  // k-chunks per batch of loads (the double-buffered fragments stay within 64 VGPRs)
  constexpr int U = (RES ? 8 : 4) / (int)(sizeof(T) / 2);
  __shared__ __align__(16) unsigned char a_lds[RES ? 16 * ASTR : 16];
  __shared__ float red[kSWaves][256];
  __shared__ float ct[256];
  __shared__ double inv_freq[64];   // RoPE inverse frequencies (head_dim <= 128)
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
  const int layer = blockIdx.y;
  if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    if (tid < a.hd / 2) inv_freq[tid] = rope_inv_freq(tid, a.hd, a.log2_theta);
    __syncthreads();
  }
  const T *W = (const T *)a.W[layer];
  const int ntiles = a.n_groups;
  const int CPT = a.K / 32;                                    // chunks per tile
  const int CPW = (CPT + kSWaves - 1) / kSWaves;               // chunks per wave
  const int cbeg = min(CPT, wave * CPW), cend = min(CPT, cbeg + CPW);
  const int nb = (CPW + U - 1) / U;                            // batches per tile per wave
  const int my_tiles = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int total = my_tiles * nb;

  const T *A = (const T *)a.A;
  const bool row_ok = ln < a.M;
  const T *arow = RES ? reinterpret_cast<const T *>(a_lds + ln * ASTR) + 8 * g
                      : A + (size_t)(row_ok ? ln : 0) * a.lda + 8 * g;
  // first weight batch goes out before the activations are staged
  StreamBuf<T, U, RES> bufa, bufb;
  if (total > 0) bufa.template issue<EPI>(a, W, arow, row_ok, blockIdx.x, cbeg, cend);

  // ---- resident activation rows ---------------------------------------------
  if constexpr (RES) {
    // wave w owns row w; one pass with the row held in registers
    constexpr int PER = KR / 64;              // elements per lane at most
    constexpr int EPV = 16 / (int)sizeof(T);  // elements per 16-byte vector
    const int r = wave;
    T *dst = reinterpret_cast<T *>(a_lds + r * ASTR);
    const int nvec = a.K / EPV;               // 16-byte vectors in the row
    if constexpr (AM == A_COPY) {
      if (r < a.M) {
        for (int i = lane; i < nvec; i += 64)
          *reinterpret_cast<uint4 *>(dst + i * EPV) = *reinterpret_cast<const uint4 *>(A + (size_t)r * a.lda + i * EPV);
      } else {
        for (int i = lane; i < nvec; i += 64) *reinterpret_cast<uint4 *>(dst + i * EPV) = make_uint4(0, 0, 0, 0);
      }
    } else {
      // lane owns elements [4*(lane + 64*j), +4) for j < K/256 (fp32 X) or the
      // same spans of the bf16 embedding row
      float v[PER];
      const int nq4 = a.K / 4;                // float4 groups in the row
      if (r < a.M) {
        if constexpr (AM == A_EMBED_NORM) {
          const int s = r / a.block_size, j = r - s * a.block_size;
          const int id = j == 0 ? a.anchor[s] : a.mask_id;
          const T *erow = (const T *)a.embed + (size_t)id * a.K;
#pragma unroll
          for (int k = 0; k < PER / 4; ++k) {
            const int q4 = lane + 64 * k;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[4 * k + e] = q4 < nq4 ? Storage<T>::load(erow, 4 * q4 + e) : 0.f;
          }
        } else {
          const float4 *x4 = reinterpret_cast<const float4 *>(a.X + (size_t)r * a.ldx);
#pragma unroll
          for (int k = 0; k < PER / 4; ++k) {
            const int q4 = lane + 64 * k;
            const float4 f = q4 < nq4 ? x4[q4] : make_float4(0.f, 0.f, 0.f, 0.f);
            v[4 * k] = f.x; v[4 * k + 1] = f.y; v[4 * k + 2] = f.z; v[4 * k + 3] = f.w;
          }
        }
        float ss = 0.f;
#pragma unroll
        for (int k = 0; k < PER; ++k) ss += v[k] * v[k];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
        const float rs = 1.0f / sqrtf(ss / (float)a.K + a.eps);
        const T *gain = (const T *)a.gain;
        const bool write_x = AM == A_EMBED_NORM && blockIdx.x == 0 && blockIdx.y == 0;
#pragma unroll
        for (int k = 0; k < PER / 4; ++k) {
          const int q4 = lane + 64 * k;
          if (q4 < nq4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int i = 4 * q4 + e;
              if (write_x) a.X[(size_t)r * a.ldx + i] = v[4 * k + e];   // residual stream
              Storage<T>::store(dst, i, v[4 * k + e] * rs * Storage<T>::load(gain, i));
            }
          }
        }
      } else {
        for (int i = lane; i < nvec; i += 64) *reinterpret_cast<uint4 *>(dst + i * EPV) = make_uint4(0, 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- weight (and activation) fragment pipeline, two batches in flight ------
  float best_v = -INFINITY;
  int best_i = 0x7fffffff;
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  // static ping-pong between two register buffers (dynamic selection would
  // spill the fragments to scratch)
  for (int q = 0; q < total; q += 2) {
    if (q + 1 < total)
      bufb.template issue<EPI>(a, W, arow, row_ok, blockIdx.x + ((q + 1) / nb) * gridDim.x,
                               cbeg + ((q + 1) % nb) * U, cend);
    acc = bufa.compute(acc, arow, cbeg + (q % nb) * U, cend);
    if (q % nb == nb - 1)
      s_finish_tile<T, EPI>(a, acc, red, ct, blockIdx.x + (q / nb) * gridDim.x, layer, &best_v, &best_i, inv_freq);
    if (q + 1 >= total) break;
    if (q + 2 < total)
      bufa.template issue<EPI>(a, W, arow, row_ok, blockIdx.x + ((q + 2) / nb) * gridDim.x,
                               cbeg + ((q + 2) % nb) * U, cend);
    acc = bufb.compute(acc, arow, cbeg + ((q + 1) % nb) * U, cend);
    if ((q + 1) % nb == nb - 1)
      s_finish_tile<T, EPI>(a, acc, red, ct, blockIdx.x + ((q + 1) / nb) * gridDim.x, layer, &best_v, &best_i, inv_freq);
  }

  if constexpr (EPI == EPI_ARGMAX) {
    if (tid < 16 && tid < a.M) {
      a.amax_val[(size_t)tid * gridDim.x + blockIdx.x] = best_v;
      a.amax_idx[(size_t)tid * gridDim.x + blockIdx.x] = best_i;
    }
  }
}

// K longer than the resident capacity: one 16-column tile per workgroup, the
// activation rows staged into LDS one K-portion at a time (each wave takes an
// even share of the portion's k-chunks); the weight fragments of the next
// batch are in flight across portion boundaries, the accumulator stays in
// registers until the whole K is done.
template <typename T, int EPI>
__global__ __launch_bounds__(kSThreads) void gemm_portion_kernel(const GemmArgs a) {
  constexpr int KR = stream_res_k<T>();
  constexpr int ASTR = KR * (int)sizeof(T) + 16;
  constexpr int U = 8 / (int)(sizeof(T) / 2);
  constexpr int EPV = 16 / (int)sizeof(T);
  __shared__ __align__(16) unsigned char a_lds[16 * ASTR];
  __shared__ float red[kSWaves][256];
  __shared__ float ct[256];
  __shared__ double inv_freq[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
  const int layer = blockIdx.y, t = blockIdx.x;
  if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    if (tid < a.hd / 2) inv_freq[tid] = rope_inv_freq(tid, a.hd, a.log2_theta);
  }
  const T *W = (const T *)a.W[layer];
  const T *A = (const T *)a.A;
  const int np = (a.K + KR - 1) / KR;               // portions
  const int CPP = KR / 32;                          // chunks per full portion
  const int CPW = (CPP + kSWaves - 1) / kSWaves;    // chunks per wave per portion
  const int nb = (CPW + U - 1) / U;                 // batches per wave per portion
  const int total = np * nb;
  const T *wrow = W + (size_t)s_weight_row<EPI>(a, t, ln) * a.ldw + 8 * g;
  const T *arow = reinterpret_cast<const T *>(a_lds + ln * ASTR) + 8 * g;
  // chunk range of unit q (portion q / nb, batch q % nb), in absolute chunks
  auto range = [&](int q, int *c0, int *c1) {
    const int p = q / nb, b = q % nb;
    const int pc = min(CPP, a.K / 32 - p * CPP);    // chunks in this portion
    const int wb = min(pc, wave * CPW), we = min(pc, wb + CPW);
    *c0 = p * CPP + min(we, wb + b * U);
    *c1 = p * CPP + min(we, wb + b * U + U);
  };
  auto stage = [&](int p) {                         // wave w copies row w of portion p
    const int r = wave;
    T *dst = reinterpret_cast<T *>(a_lds + r * ASTR);
    const int kk = min(KR, a.K - p * KR);
    for (int i = lane; i < kk / EPV; i += 64)
      *reinterpret_cast<uint4 *>(dst + i * EPV) =
          r < a.M ? *reinterpret_cast<const uint4 *>(A + (size_t)r * a.lda + p * KR + i * EPV) : make_uint4(0, 0, 0, 0);
  };
  Frag<T> wa[U], wb[U];
  int c0, c1;
  range(0, &c0, &c1);
#pragma unroll
  for (int j = 0; j < U; ++j) {
    if (c0 + j < c1) wa[j].load(wrow + 32 * (c0 + j)); else wa[j].zero();
  }
  stage(0);
  __syncthreads();
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int q = 0; q < total; q += 2) {
    // --- unit q from wa, prefetch q + 1 into wb
    int n0, n1;
    if (q + 1 < total) {
      range(q + 1, &n0, &n1);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (n0 + j < n1) wb[j].load(wrow + 32 * (n0 + j)); else wb[j].zero();
      }
    }
    range(q, &c0, &c1);
    {
      const int pbase = (q / nb) * CPP;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (c0 + j < c1) {
          Frag<T> af;
          af.load(arow + 32 * (c0 + j - pbase));
          acc = mma(acc, af, wa[j]);
        }
      }
    }
    if (q + 1 < total && (q + 1) % nb == 0) {       // next unit starts a new portion
      lds_barrier();
      stage((q + 1) / nb);
      lds_barrier();
    }
    if (q + 1 >= total) break;
    // --- unit q + 1 from wb, prefetch q + 2 into wa
    if (q + 2 < total) {
      range(q + 2, &n0, &n1);
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (n0 + j < n1) wa[j].load(wrow + 32 * (n0 + j)); else wa[j].zero();
      }
    }
    range(q + 1, &c0, &c1);
    {
      const int pbase = ((q + 1) / nb) * CPP;
#pragma unroll
      for (int j = 0; j < U; ++j) {
        if (c0 + j < c1) {
          Frag<T> af;
          af.load(arow + 32 * (c0 + j - pbase));
          acc = mma(acc, af, wb[j]);
        }
      }
    }
    if (q + 2 < total && (q + 2) % nb == 0) {
      lds_barrier();
      stage((q + 2) / nb);
      lds_barrier();
    }
  }
  float best_v = -INFINITY;
  int best_i = 0x7fffffff;
  s_finish_tile<T, EPI>(a, acc, red, ct, t, layer, &best_v, &best_i, inv_freq);
  if constexpr (EPI == EPI_ARGMAX) {
    if (tid < 16 && tid < a.M) {
      a.amax_val[(size_t)tid * gridDim.x + blockIdx.x] = best_v;
      a.amax_idx[(size_t)tid * gridDim.x + blockIdx.x] = best_i;
    }
  }
}

template <typename T, int EPI>
static hipError_t launch_s(int am, const GemmArgs &a, dim3 grid, hipStream_t st) {
  const dim3 block(kSThreads);
  switch (am) {
    case A_GLOBAL: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_GLOBAL>), grid, block, 0, st, a); break;
    case A_COPY: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_COPY>), grid, block, 0, st, a); break;
    case A_NORM: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_NORM>), grid, block, 0, st, a); break;
    case A_EMBED_NORM:
      hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_EMBED_NORM>), grid, block, 0, st, a);
      break;
    case 4:   // K-portions, one tile per workgroup (grid.x = tiles)
      hipLaunchKernelGGL((gemm_portion_kernel<T, EPI>), dim3(a.n_groups, grid.y), block, 0, st, a);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_st(Epilogue epi, int am, const GemmArgs &a, dim3 grid, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: return launch_s<T, EPI_STORE>(am, a, grid, st);
    case EPI_STORE_F32: return launch_s<T, EPI_STORE_F32>(am, a, grid, st);
    case EPI_RESID: return launch_s<T, EPI_RESID>(am, a, grid, st);
    case EPI_SWIGLU: return launch_s<T, EPI_SWIGLU>(am, a, grid, st);
    case EPI_QKV: return launch_s<T, EPI_QKV>(am, a, grid, st);
    case EPI_INJECT: return launch_s<T, EPI_INJECT>(am, a, grid, st);
    case EPI_ARGMAX: return launch_s<T, EPI_ARGMAX>(am, a, grid, st);
    default: return hipErrorInvalidValue;
  }
}

int stream_res_k(bool is_bf16) { return is_bf16 ? stream_res_k<bf16_t>() : stream_res_k<float>(); }

hipError_t launch_gemm_stream(bool is_bf16, Epilogue epi, int amode, const GemmArgs &a, int grid_x, int z_slices,
                              hipStream_t st) {
  dim3 grid(grid_x, z_slices);
  return is_bf16 ? launch_st<bf16_t>(epi, amode, a, grid, st) : launch_st<float>(epi, amode, a, grid, st);
}

}  // namespace dflash
