// LDS-tiled matrix-core GEMM for many rows (batched serving, prefill
// injection): compute-bound, bf16 x bf16 -> fp32.
//
// out[M, N] = A[M, K] * W[N, K]^T, W row-major [out, in].
//
// Block tile 128 x 128 x 64 with 4 waves in a 2 x 2 arrangement, each wave
// owning 64 x 64 outputs as 4 x 4 tiles of v_mfma_f32_16x16x32_bf16.  A and W
// tiles go global -> registers -> LDS with double buffering: the next k-step's
// global loads are in flight while the current step's 32 matrix-core products
// run, and one barrier separates the steps.  LDS rows are padded by 16 bytes so
// the 16 rows a fragment read touches fall in different banks.
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so workgroup i takes tile (i % 8) * tiles_per_xcd + i / 8; within an
// XCD consecutive tiles walk the row blocks of one column block first, so a
// weight block is fetched from HBM once and re-read from that XCD's L2.
//
// The finished 128 x 128 fp32 tile is staged through LDS for the epilogue
// (residual add, storage, SwiGLU, RoPE + q/k/v scatter, paged KV write,
// per-row argmax of the block).  SwiGLU blocks interleave 64 gate rows with
// their 64 up rows; every other epilogue uses consecutive weight rows.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kTBM = 128, kTBN = 128, kTBK = 64;
constexpr int kTThreads = 256;
constexpr int kTStride = kTBK * 2 + 16;                 // bytes per LDS row of a k-step tile
constexpr int kTStage = (kTBM + kTBN) * kTStride;       // one buffer: A rows then W rows
constexpr int kTCStride = kTBN + 4;                     // floats per epilogue row
constexpr int kTLds = (2 * kTStage > kTBM * kTCStride * 4) ? 2 * kTStage : kTBM * kTCStride * 4;

template <int EPI>
__device__ __forceinline__ int t_weight_row(const GemmArgs &a, int cb, int c) {
  if constexpr (EPI == EPI_SWIGLU) return c < 64 ? cb * 64 + c : a.ffn + cb * 64 + (c - 64);
  return cb * kTBN + c;
}

template <int EPI>
__device__ void t_epilogue(const GemmArgs &a, const float *ct, int rb, int cb, int layer) {
  using T = bf16_t;
  const int tid = threadIdx.x;
  const int row0 = rb * kTBM;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    for (int i = tid; i < kTBM * kTBN; i += kTThreads) {
      const int r = i / kTBN, c = i % kTBN, row = row0 + r;
      if (row >= a.M) continue;
      const int n = cb * kTBN + c;
      const float v = ct[r * kTCStride + c];
      if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)row * a.ldo + n, v);
      else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)row * a.ldo + n] = v;
      else a.X[(size_t)row * a.ldx + n] += v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int i = tid; i < kTBM * 64; i += kTThreads) {
      const int r = i / 64, c = i % 64, row = row0 + r;
      if (row >= a.M) continue;
      const float gt = ct[r * kTCStride + c], up = ct[r * kTCStride + 64 + c];
      Storage<T>::store((T *)a.out, (size_t)row * a.ldo + cb * 64 + c, gt / (1.0f + expf(-gt)) * up);
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int hd = a.hd, half = hd / 2;
    const int qcols = (EPI == EPI_QKV) ? a.nq * hd : 0;
    const int kcols = a.nkv * hd;
    // one thread per (row, rotation pair); pairs are (c, c + d/2) inside each head
    for (int i = tid; i < kTBM * 64; i += kTThreads) {
      const int r = i / 64, p = i % 64, row = row0 + r;
      if (row >= a.M) continue;
      const int c = (p / half) * hd + (p % half);     // lower element of the pair in the block
      const int n = cb * kTBN + c;
      const float x1 = ct[r * kTCStride + c], x2 = ct[r * kTCStride + c + half];
      int pos;
      size_t slot = 0;
      if constexpr (EPI == EPI_QKV) {
        const int s = row / a.block_size, j = row - s * a.block_size;
        pos = a.ctx_len[s] + j;
      } else {
        pos = a.pos[row];
        const int s = a.seq[row];
        const int page = a.block_table[(size_t)s * a.max_pages + pos / a.page_size];
        slot = (size_t)layer * a.cache_layer_stride + ((size_t)page * a.page_size + (pos % a.page_size)) * kcols;
      }
      float lo = x1, hi = x2;
      if (n < qcols + kcols) {
        float cs, sn;
        rope_cs_inv(pos, rope_inv_freq(p % half, hd, a.log2_theta), &cs, &sn);
        lo = x1 * cs - x2 * sn;
        hi = x2 * cs + x1 * sn;
      }
      T *dst;
      size_t off;
      if (n < qcols) {
        dst = (T *)a.q_out;
        off = (size_t)row * qcols + n;
      } else if (n < qcols + kcols) {
        dst = (T *)a.k_out;
        off = (EPI == EPI_QKV ? (size_t)row * kcols : slot) + (n - qcols);
      } else {
        dst = (T *)a.v_out;
        off = (EPI == EPI_QKV ? (size_t)row * kcols : slot) + (n - qcols - kcols);
      }
      Storage<T>::store(dst, off, lo);
      Storage<T>::store(dst, off + half, hi);
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // 2 threads per row, 64 columns each; lowest column on ties
    const int r = tid >> 1, h = tid & 1, row = row0 + r;
    float best = -INFINITY;
    int bc = 0x7fffffff;
    if (row < a.M) {
      for (int c = h * 64; c < h * 64 + 64; ++c) {
        const float v = ct[r * kTCStride + c];
        if (v > best) { best = v; bc = c; }
      }
    }
    const float ob = __shfl_xor(best, 1);
    const int oc = __shfl_xor(bc, 1);
    if (ob > best || (ob == best && oc < bc)) { best = ob; bc = oc; }
    if (h == 0 && row < a.M) {
      a.amax_val[(size_t)row * a.n_groups + cb] = best;
      a.amax_idx[(size_t)row * a.n_groups + cb] = cb * kTBN + bc;
    }
  }
}

template <int EPI>
__global__ __launch_bounds__(kTThreads) void gemm_tiled_kernel(const GemmArgs a, int n_rb, int n_cb, int per_xcd) {
  using T = bf16_t;
  __shared__ __align__(16) unsigned char lds[kTLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
  const int layer = blockIdx.y;
  // XCD-aware tile index; row blocks of a column block are consecutive
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= n_rb * n_cb) return;
  const int cb = tile / n_rb, rb = tile % n_rb;
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const int row0 = rb * kTBM;

  // global -> register staging: 4 + 4 16-byte chunks per thread per k-step
  const int crow = tid >> 3, cchunk = tid & 7;          // rows crow + 32 j, 16-byte chunk cchunk
  const T *ag = A + (size_t)row0 * a.lda + cchunk * 8;
  const T *wg = W + cchunk * 8;
  const int arows = a.M - row0;                          // valid rows of this block
  uint4 ra0, ra1, ra2, ra3, rw0, rw1, rw2, rw3;
#define DF_GLOAD(k0)                                                                                        \
  do {                                                                                                      \
    const int k_ = (k0);                                                                                    \
    ra0 = crow < arows ? *reinterpret_cast<const uint4 *>(ag + (size_t)crow * a.lda + k_) : make_uint4(0, 0, 0, 0); \
    ra1 = crow + 32 < arows ? *reinterpret_cast<const uint4 *>(ag + (size_t)(crow + 32) * a.lda + k_)       \
                            : make_uint4(0, 0, 0, 0);                                                       \
    ra2 = crow + 64 < arows ? *reinterpret_cast<const uint4 *>(ag + (size_t)(crow + 64) * a.lda + k_)       \
                            : make_uint4(0, 0, 0, 0);                                                       \
    ra3 = crow + 96 < arows ? *reinterpret_cast<const uint4 *>(ag + (size_t)(crow + 96) * a.lda + k_)       \
                            : make_uint4(0, 0, 0, 0);                                                       \
    rw0 = *reinterpret_cast<const uint4 *>(wg + (size_t)t_weight_row<EPI>(a, cb, crow) * a.ldw + k_);      \
    rw1 = *reinterpret_cast<const uint4 *>(wg + (size_t)t_weight_row<EPI>(a, cb, crow + 32) * a.ldw + k_); \
    rw2 = *reinterpret_cast<const uint4 *>(wg + (size_t)t_weight_row<EPI>(a, cb, crow + 64) * a.ldw + k_); \
    rw3 = *reinterpret_cast<const uint4 *>(wg + (size_t)t_weight_row<EPI>(a, cb, crow + 96) * a.ldw + k_); \
  } while (0)
#define DF_LSTORE(buf)                                                                                      \
  do {                                                                                                      \
    unsigned char *b_ = lds + (buf) * kTStage + crow * kTStride + cchunk * 16;                              \
    *reinterpret_cast<uint4 *>(b_) = ra0;                                                                   \
    *reinterpret_cast<uint4 *>(b_ + 32 * kTStride) = ra1;                                                   \
    *reinterpret_cast<uint4 *>(b_ + 64 * kTStride) = ra2;                                                   \
    *reinterpret_cast<uint4 *>(b_ + 96 * kTStride) = ra3;                                                   \
    *reinterpret_cast<uint4 *>(b_ + kTBM * kTStride) = rw0;                                                 \
    *reinterpret_cast<uint4 *>(b_ + (kTBM + 32) * kTStride) = rw1;                                          \
    *reinterpret_cast<uint4 *>(b_ + (kTBM + 64) * kTStride) = rw2;                                          \
    *reinterpret_cast<uint4 *>(b_ + (kTBM + 96) * kTStride) = rw3;                                          \
  } while (0)

  const int wr = wave >> 1, wc = wave & 1;               // wave's 64 x 64 quadrant
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = a.K / kTBK;
  DF_GLOAD(0);
  DF_LSTORE(0);
  __syncthreads();
  for (int kt = 0; kt < nk; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nk) DF_GLOAD((kt + 1) * kTBK);
    const unsigned char *base = lds + buf * kTStage;
#pragma unroll
    for (int kc = 0; kc < 2; ++kc) {
      Frag<T> af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        af[i].load(reinterpret_cast<const T *>(base + (wr * 64 + i * 16 + ln) * kTStride) + kc * 32 + 8 * g);
        bf[i].load(reinterpret_cast<const T *>(base + (kTBM + wc * 64 + i * 16 + ln) * kTStride) + kc * 32 + 8 * g);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mma(acc[i][j], af[i], bf[j]);
    }
    if (kt + 1 < nk) DF_LSTORE(buf ^ 1);
    __syncthreads();
  }

  // stage the fp32 tile through LDS (the k-step buffers are no longer read)
  float *ct = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        ct[(wr * 64 + i * 16 + 4 * g + e) * kTCStride + wc * 64 + j * 16 + ln] = f4get(acc[i][j], e);
  __syncthreads();
  t_epilogue<EPI>(a, ct, rb, cb, layer);
}
#undef DF_GLOAD
#undef DF_LSTORE

int gemm_tiled_cols(Epilogue epi, int N, int ffn) { return epi == EPI_SWIGLU ? ffn / 64 : N / kTBN; }

bool gemm_tiled_ok(Epilogue epi, int N, int K, int ffn, int hd) {
  if (K % kTBK) return false;
  if (epi == EPI_SWIGLU) return ffn % 64 == 0;
  if ((epi == EPI_QKV || epi == EPI_INJECT) && kTBN % hd) return false;
  return N % kTBN == 0;
}

hipError_t launch_gemm_tiled(Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  const int n_rb = (a.M + kTBM - 1) / kTBM;
  const int n_cb = a.n_groups;
  const int per_xcd = (n_rb * n_cb + 7) / 8;
  dim3 grid(8 * per_xcd, z_slices), block(kTThreads);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL(gemm_tiled_kernel<EPI_STORE>, grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_STORE_F32:
      hipLaunchKernelGGL(gemm_tiled_kernel<EPI_STORE_F32>, grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_RESID: hipLaunchKernelGGL(gemm_tiled_kernel<EPI_RESID>, grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL(gemm_tiled_kernel<EPI_SWIGLU>, grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_QKV: hipLaunchKernelGGL(gemm_tiled_kernel<EPI_QKV>, grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_INJECT:
      hipLaunchKernelGGL(gemm_tiled_kernel<EPI_INJECT>, grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL(gemm_tiled_kernel<EPI_ARGMAX>, grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace dflash
