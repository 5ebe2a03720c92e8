// Weight-streaming matrix-core GEMM for few rows (the drafter's projections at
// small batch) with fused epilogues.
//
// out[M, N] = A[M, K] * W[N, K]^T, W row-major [out, in] as stored.
//
// Work decomposition.  A workgroup (4 waves) owns 128 output columns, up to 64
// rows and a slice of K.  Wave w owns column tiles {w, w+4} of the group, i.e.
// local columns 16w..16w+15 and 64+16w..64+16w+15, so a 128-wide group holds
// one full head (RoPE partners i and i+64 for head_dim 128) or, for SwiGLU, 64
// gate columns beside their 64 up columns.  The activations of the K slice are
// staged once per stage in LDS (they are tiny and shared by the 4 waves); the
// weights stream from HBM straight into matrix-core fragments, 8 k-chunks per
// batch of loads, with no LDS round trip.
//
// Split-K.  When there are too few column groups to fill the chip, K is cut
// into k_split slices.  Each slice stores its fp32 partial tile; the workgroup
// that arrives last at the group's counter sums the partials in slice order
// (deterministic) and runs the epilogue.  The counter is reset by that
// workgroup, so no clearing launch is needed between calls.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

template <typename T, int MT>
struct GemmShape {
  static constexpr int MP = 16 * MT;                                // rows per workgroup
  static constexpr int KS = 32768 / (MP * (int)sizeof(T));          // k-elements per LDS stage
  static constexpr int A_STRIDE = KS * (int)sizeof(T) + 16;         // bytes per staged row
  static constexpr int A_BYTES = MP * A_STRIDE;
  static constexpr int C_STRIDE = kColGroup + 4;                    // floats per epilogue row
  static constexpr int C_BYTES = MP * C_STRIDE * 4;
  static constexpr int LDS = A_BYTES > C_BYTES ? A_BYTES : C_BYTES;
};

int gemm_rows_per_group(int M) { return M <= 16 ? 16 : (M <= 32 ? 32 : 64); }

size_t gemm_plan(int M, int n_groups, int K, int z_slices, bool is_bf16, int *k_split, int *k_per_split) {
  const int MP = gemm_rows_per_group(M);
  const int m_groups = (M + MP - 1) / MP;
  const long blocks = (long)n_groups * z_slices * m_groups;
  const int max_split = K / 256 > 1 ? K / 256 : 1;
  long want = (2048 + blocks - 1) / blocks;
  int ks = (int)(want < 1 ? 1 : (want > max_split ? max_split : want));
  int kps = (K + ks - 1) / ks;
  kps = (kps + 31) / 32 * 32;
  ks = (K + kps - 1) / kps;
  (void)is_bf16;
  *k_split = ks;
  *k_per_split = kps;
  return ks > 1 ? (size_t)z_slices * m_groups * n_groups * ks * MP * kColGroup : 0;
}

// Physical weight row of local column lc of column group cg (and its validity).
template <int EPI>
__device__ __forceinline__ int weight_row(const GemmArgs &a, int cg, int lc, bool *valid) {
  if (EPI == EPI_SWIGLU) {
    const int j = cg * 64 + (lc & 63);
    *valid = j < a.ffn;
    return lc < 64 ? j : a.ffn + j;
  }
  const int n = cg * kColGroup + lc;
  *valid = n < a.N;
  return n;
}

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs &a, const float *ct, int c_stride, int MP, int row0, int cg,
                              int layer) {
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    for (int i = tid; i < MP * kColGroup; i += blockDim.x) {
      const int r = i / kColGroup, c = i % kColGroup;
      const int row = row0 + r, n = cg * kColGroup + c;
      if (row >= a.M || n >= a.N) continue;
      const float v = ct[r * c_stride + c];
      if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)row * a.ldo + n, v);
      else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)row * a.ldo + n] = v;
      else a.X[(size_t)row * a.ldx + n] += v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int i = tid; i < MP * 64; i += blockDim.x) {
      const int r = i / 64, c = i % 64;
      const int row = row0 + r, j = cg * 64 + c;
      if (row >= a.M || j >= a.ffn) continue;
      const float gt = ct[r * c_stride + c], up = ct[r * c_stride + 64 + c];
      const float silu = gt / (1.0f + expf(-gt));
      Storage<T>::store((T *)a.out, (size_t)row * a.ldo + j, silu * up);
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    // one thread per rotation pair (i, i + hd/2) or per value element
    const int hd = a.hd, half = hd / 2;
    const int qcols = (EPI == EPI_QKV) ? a.nq * hd : 0;
    const int kcols = a.nkv * hd;
    for (int i = tid; i < MP * kColGroup; i += blockDim.x) {
      const int r = i / kColGroup, c = i % kColGroup;
      const int row = row0 + r, n = cg * kColGroup + c;
      if (row >= a.M || n >= a.N) continue;
      int pos;
      size_t dst_k = 0, dst_v = 0;
      if constexpr (EPI == EPI_QKV) {
        const int s = row / a.block_size, j = row % a.block_size;
        pos = a.ctx_len[s] + j;
      } else {
        pos = a.pos[row];
        const int s = a.seq[row];
        const int page = a.block_table[(size_t)s * a.max_pages + pos / a.page_size];
        const size_t slot = ((size_t)page * a.page_size + (pos % a.page_size)) * (size_t)kcols;
        dst_k = (size_t)layer * a.cache_layer_stride + slot;
        dst_v = dst_k;
      }
      const float x = ct[r * c_stride + c];
      if (n < qcols + kcols) {
        // rotary pair: only the lower element's thread writes both
        const int within = (n - (n < qcols ? 0 : qcols)) % hd;
        if (within >= half) continue;
        const float x2 = ct[r * c_stride + c + half];
        float cs, sn;
        rope_cs(pos, within, hd, a.log2_theta, &cs, &sn);
        const float lo = x * cs - x2 * sn, hi = x2 * cs + x * sn;
        if (n < qcols) {
          T *q = (T *)a.q_out;
          Storage<T>::store(q, (size_t)row * qcols + n, lo);
          Storage<T>::store(q, (size_t)row * qcols + n + half, hi);
        } else {
          const int kn = n - qcols;
          if constexpr (EPI == EPI_QKV) {
            T *k = (T *)a.k_out;
            Storage<T>::store(k, (size_t)row * kcols + kn, lo);
            Storage<T>::store(k, (size_t)row * kcols + kn + half, hi);
          } else {
            T *k = (T *)a.k_out;
            Storage<T>::store(k, dst_k + kn, lo);
            Storage<T>::store(k, dst_k + kn + half, hi);
          }
        }
      } else {
        const int vn = n - qcols - kcols;
        if constexpr (EPI == EPI_QKV) Storage<T>::store((T *)a.v_out, (size_t)row * kcols + vn, x);
        else Storage<T>::store((T *)a.v_out, dst_v + vn, x);
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // 4 threads per row, 32 columns each; lowest column wins ties
    const int r = tid >> 2, q = tid & 3;
    float best = -INFINITY;
    int bidx = 0x7fffffff;
    if (r < MP && row0 + r < a.M) {
      for (int c = q * 32; c < q * 32 + 32; ++c) {
        const int n = cg * kColGroup + c;
        if (n >= a.N) break;
        const float v = ct[r * c_stride + c];
        if (v > best) { best = v; bidx = n; }
      }
    }
#pragma unroll
    for (int m = 1; m <= 2; m <<= 1) {
      const float ov = __shfl_xor(best, m);
      const int oi = __shfl_xor(bidx, m);
      if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
    }
    if (q == 0 && r < MP && row0 + r < a.M) {
      a.amax_val[(size_t)(row0 + r) * a.n_groups + cg] = best;
      a.amax_idx[(size_t)(row0 + r) * a.n_groups + cg] = bidx;
    }
  }
}

template <typename T, int MT, int EPI>
__global__ __launch_bounds__(256) void gemm_kernel(const GemmArgs a) {
  using S = GemmShape<T, MT>;
  __shared__ __align__(16) unsigned char smem[S::LDS];
  __shared__ int last_flag;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4;
  const int cg = blockIdx.x, ks = blockIdx.y;
  const int layer = blockIdx.z / a.m_groups, mg = blockIdx.z % a.m_groups;
  const int row0 = mg * S::MP;
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const int k_begin = ks * a.k_per_split;
  const int k_end = min(a.K, k_begin + a.k_per_split);

  bool v0, v1;
  const int r0 = weight_row<EPI>(a, cg, 16 * wave + (lane & 15), &v0);
  const int r1 = weight_row<EPI>(a, cg, 64 + 16 * wave + (lane & 15), &v1);
  const T *w0 = W + (size_t)(v0 ? r0 : 0) * a.ldw + 8 * g;
  const T *w1 = W + (size_t)(v1 ? r1 : 0) * a.ldw + 8 * g;

  f32x4 acc[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt][0] = acc[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int kb = k_begin; kb < k_end; kb += S::KS) {
    const int kn = min(S::KS, k_end - kb);
    __syncthreads();
    constexpr int EPV = 16 / (int)sizeof(T);
    const int vpr = kn / EPV;
    for (int i = tid; i < S::MP * vpr; i += 256) {
      const int r = i / vpr, cv = i - r * vpr;
      uint4 val = make_uint4(0, 0, 0, 0);
      if (row0 + r < a.M) val = *reinterpret_cast<const uint4 *>(A + (size_t)(row0 + r) * a.lda + kb + cv * EPV);
      *reinterpret_cast<uint4 *>(smem + r * S::A_STRIDE + cv * 16) = val;
    }
    __syncthreads();
    const T *arow = reinterpret_cast<const T *>(smem + (lane & 15) * S::A_STRIDE) + 8 * g;
    const int nchunk = kn / 32;
    int u = 0;
    for (; u + 8 <= nchunk; u += 8) {
      Frag<T> b0[8], b1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (v0) b0[j].load(w0 + kb + 32 * (u + j)); else b0[j].zero();
        if (v1) b1[j].load(w1 + kb + 32 * (u + j)); else b1[j].zero();
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Frag<T> af;
          af.load(reinterpret_cast<const T *>(reinterpret_cast<const unsigned char *>(arow) + mt * 16 * S::A_STRIDE) +
                  32 * (u + j));
          acc[mt][0] = mma(acc[mt][0], af, b0[j]);
          acc[mt][1] = mma(acc[mt][1], af, b1[j]);
        }
      }
    }
    for (; u < nchunk; ++u) {
      Frag<T> b0, b1;
      if (v0) b0.load(w0 + kb + 32 * u); else b0.zero();
      if (v1) b1.load(w1 + kb + 32 * u); else b1.zero();
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        Frag<T> af;
        af.load(reinterpret_cast<const T *>(reinterpret_cast<const unsigned char *>(arow) + mt * 16 * S::A_STRIDE) +
                32 * u);
        acc[mt][0] = mma(acc[mt][0], af, b0);
        acc[mt][1] = mma(acc[mt][1], af, b1);
      }
    }
  }

  float *ct = reinterpret_cast<float *>(smem);
  const int tile_tot = S::MP * kColGroup;
  if (a.k_split == 1) {
    __syncthreads();  // all waves finished reading the staged activations
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = t * 64 + 16 * wave + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) ct[(mt * 16 + 4 * g + i) * S::C_STRIDE + c] = f4get(acc[mt][t], i);
      }
  } else {
    const size_t grp = (size_t)blockIdx.z * a.n_groups + cg;
    float *part = a.partial + (grp * a.k_split + ks) * tile_tot;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int c = t * 64 + 16 * wave + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) part[(mt * 16 + 4 * g + i) * kColGroup + c] = f4get(acc[mt][t], i);
      }
    if (!arrive_last(a.counters + grp, a.k_split, &last_flag)) return;
    const float *base = a.partial + grp * a.k_split * tile_tot;
    for (int i = tid; i < tile_tot; i += 256) {
      float s = 0.f;
      for (int kk = 0; kk < a.k_split; ++kk) s += base[(size_t)kk * tile_tot + i];
      ct[(i / kColGroup) * S::C_STRIDE + (i % kColGroup)] = s;
    }
  }
  __syncthreads();
  gemm_epilogue<T, EPI>(a, ct, S::C_STRIDE, S::MP, row0, cg, layer);
}

template <typename T, int MT>
static hipError_t launch_mt(Epilogue epi, const GemmArgs &a, dim3 grid, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_STORE>), grid, dim3(256), 0, st, a); break;
    case EPI_STORE_F32: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_STORE_F32>), grid, dim3(256), 0, st, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_RESID>), grid, dim3(256), 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_SWIGLU>), grid, dim3(256), 0, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_QKV>), grid, dim3(256), 0, st, a); break;
    case EPI_INJECT: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_INJECT>), grid, dim3(256), 0, st, a); break;
    case EPI_ARGMAX: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_ARGMAX>), grid, dim3(256), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(bool is_bf16, Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  const int MP = gemm_rows_per_group(a.M);
  dim3 grid(a.n_groups, a.k_split, z_slices * a.m_groups);
  if (is_bf16) {
    if (MP == 16) return launch_mt<bf16_t, 1>(epi, a, grid, st);
    if (MP == 32) return launch_mt<bf16_t, 2>(epi, a, grid, st);
    return launch_mt<bf16_t, 4>(epi, a, grid, st);
  }
  if (MP == 16) return launch_mt<float, 1>(epi, a, grid, st);
  if (MP == 32) return launch_mt<float, 2>(epi, a, grid, st);
  return launch_mt<float, 4>(epi, a, grid, st);
}

}  // namespace dflash
