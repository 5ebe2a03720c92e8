// LDS-tiled matrix-core GEMM for many rows (batched serving, prefill
// injection): compute-bound, bf16 x bf16 -> fp32.
//
// out[M, N] = A[M, K] * W[N, K]^T, W row-major [out, in].
//
// Block tile BM x 128 x 64 (BM = 128 or 256) with BM/64 x 2 waves, each wave
// owning a 64 x 64 quadrant as 2 x 2 tiles of v_mfma_f32_32x32x16_bf16 (half
// the LDS reads per flop of 16 x 16 tiles; lane l supplies row l % 32 and the
// 8 k-elements 8*(l/32).. of each operand, and holds column l % 32, rows
// 8*(i/4) + 4*(l/32) + i%4 of the result).
//
// Staging: k-step tiles go from global memory straight into LDS with
// LDS-direct loads (no registers), through a ring of three stages; two stages
// are always in flight while the third is multiplied, so every wait is "all
// but the last stage's loads".  An instruction moves 1 KB = 8 rows of 64
// k-elements; lane l fills row l/8, 16-byte slot l%8, and loads the global
// chunk slot ^ ((row / 2) % 8) there: a 128-byte row spans half the banks, so
// the 16 consecutive rows a fragment read serves at once (8 even rows in one
// half, 8 odd rows in the other) put their 16-byte pieces on distinct banks.  Rows past M read row M-1 (never stored).
//
// Tile order is XCD-aware: workgroups are dispatched round-robin over the 8
// XCDs, so workgroup i takes tile (i % 8) * tiles_per_xcd + i / 8; within an
// XCD consecutive tiles walk the row blocks of one column block first, so a
// weight block is fetched from HBM once and re-read from that XCD's L2.
//
// The finished fp32 tile is staged through LDS for the epilogue (residual
// add, storage, SwiGLU, RoPE + q/k/v scatter, paged KV write, per-row argmax
// of the block).  SwiGLU blocks interleave 64 gate rows with their 64 up
// rows; every other epilogue uses consecutive weight rows.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kTBN = 128, kTBK = 64;
constexpr int kTRow = kTBK * 2;                          // bytes per staged row (64 bf16)
constexpr int kTCStride = kTBN + 4;                      // floats per epilogue row
constexpr int kTStages = 3;

template <int BM> struct TCfg {
  static constexpr int waves = BM / 64 * 2;
  static constexpr int threads = waves * 64;
  static constexpr int stage = (BM + kTBN) * kTRow;      // bytes of one stage (A rows, then W rows)
  static constexpr int pieces = stage / 1024;            // 1 KB LDS-direct loads per stage
  static constexpr int per_wave = pieces / waves;        // ... per wave
  static constexpr int lds = kTStages * stage > BM * kTCStride * 4 ? kTStages * stage : BM * kTCStride * 4;
  static_assert(pieces % waves == 0, "stage pieces split evenly over the waves");
};

template <int EPI>
__device__ __forceinline__ int t_weight_row(const GemmArgs &a, int cb, int c) {
  if constexpr (EPI == EPI_SWIGLU) return c < 64 ? cb * 64 + c : a.ffn + cb * 64 + (c - 64);
  return cb * kTBN + c;
}

template <int EPI, int BM>
__device__ void t_epilogue(const GemmArgs &a, const float *ct, int rb, int cb, int layer) {
  using T = bf16_t;
  constexpr int NT = TCfg<BM>::threads;
  const int tid = threadIdx.x;
  const int row0 = rb * BM;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    for (int i = tid; i < BM * kTBN; i += NT) {
      const int r = i / kTBN, c = i % kTBN, row = row0 + r;
      if (row >= a.M) continue;
      const int n = cb * kTBN + c;
      const float v = ct[r * kTCStride + c];
      if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)row * a.ldo + n, v);
      else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)row * a.ldo + n] = v;
      else a.X[(size_t)row * a.ldx + n] += v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int i = tid; i < BM * 64; i += NT) {
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
    for (int i = tid; i < BM * 64; i += NT) {
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

template <int EPI, int BM>
__global__ __launch_bounds__(TCfg<BM>::threads) void gemm_tiled_kernel(const GemmArgs a, int n_rb, int n_cb,
                                                                       int per_xcd) {
  using T = bf16_t;
  using C = TCfg<BM>;
  __shared__ __align__(16) unsigned char lds[C::lds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int layer = blockIdx.y;
  // XCD-aware tile index; row blocks of a column block are consecutive
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= n_rb * n_cb) return;
  const int cb = tile / n_rb, rb = tile % n_rb;
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const int row0 = rb * BM;

  // LDS-direct staging: piece q of a stage covers staged rows 8q .. 8q+7
  // (A rows first, then W rows); this lane fills row 8q + lane/8, slot lane%8
  const T *src[C::per_wave];
#pragma unroll
  for (int i = 0; i < C::per_wave; ++i) {
    const int q = wave * C::per_wave + i, r = 8 * q + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    src[i] = r < BM ? A + (size_t)min(row0 + r, a.M - 1) * a.lda + chunk * 8
                    : W + (size_t)t_weight_row<EPI>(a, cb, r - BM) * a.ldw + chunk * 8;
  }
  const int nk = a.K / kTBK;
  // stage kt (clamped to the last k-step: past the end the loads are repeated
  // into a free buffer and never read)
  const unsigned lds0 = lds_offset(lds);
#define DF_STAGE(kt)                                                                                \
  do {                                                                                              \
    const int k_ = min((kt), nk - 1) * kTBK, b_ = (kt) % kTStages;                                  \
    _Pragma("unroll") for (int i = 0; i < C::per_wave; ++i)                                         \
      lds_dma16(src[i] + k_, lds0 + b_ * C::stage + (wave * C::per_wave + i) * 1024);               \
  } while (0)

  const int wr = wave >> 1, wc = wave & 1;               // wave's 64 x 64 quadrant
  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // fragment rows of this lane and their swizzle
  const int fr = lane & 31, fk = lane >> 5;              // row within a 32-tile, 8-element k group
  DF_STAGE(0);
  DF_STAGE(1);
  for (int kt = 0; kt < nk; ++kt) {
    // stage kt has landed once only the next stage's loads are outstanding;
    // the barrier also frees buffer (kt + 2) % 3, last read at step kt - 1
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(C::per_wave));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    DF_STAGE(kt + 2);
    const unsigned char *base = lds + (kt % kTStages) * C::stage;
#pragma unroll
    for (int s = 0; s < kTBK / 16; ++s) {
      Frag<T> af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int ra = wr * 64 + i * 32 + fr, rw = BM + wc * 64 + i * 32 + fr;
        const int ch = 2 * s + fk;
        af[i].v = *reinterpret_cast<const uint4 *>(base + ra * kTRow + ((ch ^ ((ra >> 1) & 7)) << 4));
        bf[i].v = *reinterpret_cast<const uint4 *>(base + rw * kTRow + ((ch ^ ((rw >> 1) & 7)) << 4));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = mma32(acc[i][j], af[i], bf[j]);
    }
  }
#undef DF_STAGE
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // stage the fp32 tile through LDS (the k-step buffers are no longer read)
  float *ct = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e)
        ct[(wr * 64 + i * 32 + 8 * (e / 4) + 4 * fk + e % 4) * kTCStride + wc * 64 + j * 32 + fr] = acc[i][j][e];
  __syncthreads();
  t_epilogue<EPI, BM>(a, ct, rb, cb, layer);
}

int gemm_tiled_cols(Epilogue epi, int N, int ffn) { return epi == EPI_SWIGLU ? ffn / 64 : N / kTBN; }

bool gemm_tiled_ok(Epilogue epi, int N, int K, int ffn, int hd) {
  if (K % kTBK) return false;
  if (epi == EPI_SWIGLU) return ffn % 64 == 0;
  if ((epi == EPI_QKV || epi == EPI_INJECT) && kTBN % hd) return false;
  return N % kTBN == 0;
}

template <int BM>
static hipError_t launch_tiled_bm(Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  const int n_rb = (a.M + BM - 1) / BM;
  const int n_cb = a.n_groups;
  const int per_xcd = (n_rb * n_cb + 7) / 8;
  dim3 grid(8 * per_xcd, z_slices), block(TCfg<BM>::threads);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_tiled_kernel<EPI_STORE, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_STORE_F32:
      hipLaunchKernelGGL((gemm_tiled_kernel<EPI_STORE_F32, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_tiled_kernel<EPI_RESID, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_SWIGLU:
      hipLaunchKernelGGL((gemm_tiled_kernel<EPI_SWIGLU, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_tiled_kernel<EPI_QKV, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd); break;
    case EPI_INJECT:
      hipLaunchKernelGGL((gemm_tiled_kernel<EPI_INJECT, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    case EPI_ARGMAX:
      hipLaunchKernelGGL((gemm_tiled_kernel<EPI_ARGMAX, BM>), grid, block, 0, st, a, n_rb, n_cb, per_xcd);
      break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// 256-row tiles when they still give a few waves of workgroups per compute
// unit; 128-row tiles otherwise (more tiles for the narrow projections).
hipError_t launch_gemm_tiled(Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  const long tiles256 = (long)((a.M + 255) / 256) * a.n_groups * z_slices;
  if (tiles256 >= 512) return launch_tiled_bm<256>(epi, a, z_slices, st);
  return launch_tiled_bm<128>(epi, a, z_slices, st);
}

}  // namespace dflash
