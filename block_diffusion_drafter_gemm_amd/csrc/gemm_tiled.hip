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
#ifndef DF_BIG_MIN_TILES
#define DF_BIG_MIN_TILES 160
#endif
constexpr int kBigMinTiles = DF_BIG_MIN_TILES;   // 256 x 256 tiles from this many tiles on

template <int BM> struct TCfg {
  static constexpr int waves = BM / 64 * 2;
  static constexpr int threads = waves * 64;
  static constexpr int stage = (BM + kTBN) * kTRow;      // bytes of one stage (A rows, then W rows)
  static constexpr int pieces = stage / 1024;            // 1 KB LDS-direct loads per stage
  static constexpr int per_wave = pieces / waves;        // ... per wave
  static constexpr int lds = kTStages * stage > BM * kTCStride * 4 ? kTStages * stage : BM * kTCStride * 4;
  static_assert(pieces % waves == 0, "stage pieces split evenly over the waves");
  static_assert(lds >= BM * kTCStride * 4 + BM * 12, "epilogue row metadata fits past the fp32 tile");
};

template <int EPI>
__device__ __forceinline__ int t_weight_row(const GemmArgs &a, int cb, int c) {
  if constexpr (EPI == EPI_SWIGLU) return c < 64 ? cb * 64 + c : a.ffn + cb * 64 + (c - 64);
  return cb * kTBN + c;
}

// Per-row metadata of the RoPE epilogues, one row per thread (threads past BM
// hold nothing): the row's position and, for the paged cache, its slot (page
// from the block table).  Loaded at kernel start, so that the dependent
// position -> page lookup is hidden behind the k-loop.
struct RowMeta {
  int pos;
  size_t slot;
};
template <int EPI, int BM>
__device__ __forceinline__ RowMeta load_row_meta(const GemmArgs &a, int row0, int layer) {
  RowMeta m{0, 0};
  if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int tid = threadIdx.x;
    if (tid < BM) {
      const int row = min(row0 + tid, a.M - 1);
      if constexpr (EPI == EPI_QKV) {
        const int s = row / a.block_size;
        m.pos = a.ctx_len[s] + (row - s * a.block_size);
      } else {
        const int pos = a.pos[row], s = a.seq[row];
        const int page = a.block_table[(size_t)s * a.max_pages + pos / a.page_size];
        m.pos = pos;
        m.slot = (size_t)layer * a.cache_layer_stride +
                 ((size_t)page * a.page_size + (pos % a.page_size)) * (size_t)(a.nkv * a.hd);
      }
    }
  }
  return m;
}

// Epilogue of a BM x 128 fp32 tile in LDS (row stride kTCStride), run by NT
// threads.  `meta` is this thread's row metadata (RoPE epilogues); `first` is
// false on the second 128-column half of the same rows, whose metadata is
// already in LDS.
template <int EPI, int BM, int NT>
__device__ void t_epilogue(const GemmArgs &a, const float *ct, int rb, int cb, int layer, const RowMeta &meta,
                           bool first) {
  using T = bf16_t;
  const int tid = threadIdx.x;
  const int row0 = rb * BM;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    // 8 consecutive columns per thread and iteration, moved as 16-byte pieces
    // when the output rows allow it (row stride and base aligned), else one
    // element at a time
    const bool vec = EPI == EPI_RESID ? (a.ldx % 4 == 0 && reinterpret_cast<uintptr_t>(a.X) % 16 == 0)
                                      : (a.ldo % (EPI == EPI_STORE ? 8 : 4) == 0 &&
                                         reinterpret_cast<uintptr_t>(a.out) % 16 == 0);
    if (vec) {
      for (int i = tid; i < BM * (kTBN / 8); i += NT) {
        const int r = i / (kTBN / 8), c = (i % (kTBN / 8)) * 8, row = row0 + r;
        if (row >= a.M) break;
        const int n = cb * kTBN + c;
        const float4 v0 = *reinterpret_cast<const float4 *>(ct + r * kTCStride + c);
        const float4 v1 = *reinterpret_cast<const float4 *>(ct + r * kTCStride + c + 4);
        if constexpr (EPI == EPI_STORE) {
          const float f[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
          Frag<T> o;
          o.set(f);
          o.store((T *)a.out + (size_t)row * a.ldo + n);
        } else if constexpr (EPI == EPI_STORE_F32) {
          float4 *o = reinterpret_cast<float4 *>((float *)a.out + (size_t)row * a.ldo + n);
          o[0] = v0;
          o[1] = v1;
        } else {
          float4 *x = reinterpret_cast<float4 *>(a.X + (size_t)row * a.ldx + n);
          float4 x0 = x[0], x1 = x[1];
          x0.x += v0.x; x0.y += v0.y; x0.z += v0.z; x0.w += v0.w;
          x1.x += v1.x; x1.y += v1.y; x1.z += v1.z; x1.w += v1.w;
          x[0] = x0;
          x[1] = x1;
        }
      }
    } else {
      for (int i = tid; i < BM * kTBN; i += NT) {
        const int r = i / kTBN, c = i % kTBN, row = row0 + r;
        if (row >= a.M) continue;
        const int n = cb * kTBN + c;
        const float v = ct[r * kTCStride + c];
        if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)row * a.ldo + n, v);
        else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)row * a.ldo + n] = v;
        else a.X[(size_t)row * a.ldx + n] += v;
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    const bool vec = a.ldo % 8 == 0 && reinterpret_cast<uintptr_t>(a.out) % 16 == 0;
    if (vec) {
      // gate columns 0..63 of the block, their up columns 64..127: 8 outputs per thread
      for (int i = tid; i < BM * 8; i += NT) {
        const int r = i / 8, c = (i % 8) * 8, row = row0 + r;
        if (row >= a.M) break;
        const float *g = ct + r * kTCStride + c, *u = g + 64;
        const float4 g0 = *reinterpret_cast<const float4 *>(g), g1 = *reinterpret_cast<const float4 *>(g + 4);
        const float4 u0 = *reinterpret_cast<const float4 *>(u), u1 = *reinterpret_cast<const float4 *>(u + 4);
        const float f[8] = {silu_mul(g0.x, u0.x), silu_mul(g0.y, u0.y), silu_mul(g0.z, u0.z), silu_mul(g0.w, u0.w),
                            silu_mul(g1.x, u1.x), silu_mul(g1.y, u1.y), silu_mul(g1.z, u1.z), silu_mul(g1.w, u1.w)};
        Frag<T> o;
        o.set(f);
        o.store((T *)a.out + (size_t)row * a.ldo + cb * 64 + c);
      }
    } else {
      for (int i = tid; i < BM * 64; i += NT) {
        const int r = i / 64, c = i % 64, row = row0 + r;
        if (row >= a.M) continue;
        const float gt = ct[r * kTCStride + c], up = ct[r * kTCStride + 64 + c];
        Storage<T>::store((T *)a.out, (size_t)row * a.ldo + cb * 64 + c, silu_mul(gt, up));
      }
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int hd = a.hd, half = hd / 2;
    const int qcols = (EPI == EPI_QKV) ? a.nq * hd : 0;
    const int kcols = a.nkv * hd;
    // row metadata into LDS past the fp32 tile, once per tile
    int *mpos = reinterpret_cast<int *>(const_cast<float *>(ct) + BM * kTCStride);
    size_t *mslot = reinterpret_cast<size_t *>(mpos + BM);
    if (first) {
      if (tid < BM) {
        mpos[tid] = meta.pos;
        mslot[tid] = meta.slot;
      }
      __syncthreads();
    }
    // One thread per (row, 8 consecutive rotation pairs): pairs are (c, c + d/2)
    // inside each head, so the thread reads 8 consecutive lower and 8 upper
    // elements and writes each group as one 16-byte piece.  NT is a multiple
    // of 8, so a thread's pairs, and their frequencies, are fixed.
    static_assert(NT % 8 == 0, "fixed pair group per thread");
    const int q = tid % 8, p0 = 8 * q;                   // pairs p0 .. p0 + 7 of the block's 64
    const int c0 = (p0 / half) * hd + (p0 % half);       // lower element of pair p0 (half % 8 == 0)
    const int n = cb * kTBN + c0;
    const bool rot = n < qcols + kcols;
    double inv_freq[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) inv_freq[k] = rope_inv_freq((p0 + k) % half, hd, a.log2_theta);
    T *dst;
    size_t coff, rstride = 0;
    if (n < qcols) {
      dst = (T *)a.q_out;
      coff = n;
      rstride = qcols;
    } else if (n < qcols + kcols) {
      dst = (T *)a.k_out;
      coff = n - qcols;
      rstride = kcols;
    } else {
      dst = (T *)a.v_out;
      coff = n - qcols - kcols;
      rstride = kcols;
    }
    for (int r = tid / 8; r < BM; r += NT / 8) {
      const int row = row0 + r;
      if (row >= a.M) break;
      const float *lp = ct + r * kTCStride + c0, *hp = lp + half;
      const float4 l0 = *reinterpret_cast<const float4 *>(lp), l1 = *reinterpret_cast<const float4 *>(lp + 4);
      const float4 h0 = *reinterpret_cast<const float4 *>(hp), h1 = *reinterpret_cast<const float4 *>(hp + 4);
      float lo[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
      float hi[8] = {h0.x, h0.y, h0.z, h0.w, h1.x, h1.y, h1.z, h1.w};
      if (rot) {
        const int pos = mpos[r];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float cs, sn;
          rope_cs_inv(pos, inv_freq[k], &cs, &sn);
          const float x1 = lo[k], x2 = hi[k];
          lo[k] = x1 * cs - x2 * sn;
          hi[k] = x2 * cs + x1 * sn;
        }
      }
      const size_t off = (EPI == EPI_QKV ? (size_t)row * rstride : mslot[r]) + coff;
      Frag<T> fl, fh;
      fl.set(lo);
      fh.set(hi);
      fl.store(dst + off);
      fh.store(dst + off + half);
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // 2 threads per row, 64 columns each; lowest column on ties (a NaN never
    // wins; no number above -inf leaves each half's first column)
    static_assert(BM % (NT / 2) == 0, "whole passes of NT / 2 rows");
    for (int r0 = 0; r0 < BM; r0 += NT / 2) {
      const int r = r0 + (tid >> 1), h = tid & 1, row = row0 + r;
      float best = -INFINITY;
      int bc = h * 64;
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
  const int kz = blockIdx.z, kbase = kz * a.kper;        // split-K: this workgroup's K range
  const RowMeta meta = load_row_meta<EPI, BM>(a, row0, layer);

  // LDS-direct staging: piece q of a stage covers staged rows 8q .. 8q+7
  // (A rows first, then W rows); this lane fills row 8q + lane/8, slot lane%8
  const T *src[C::per_wave];
#pragma unroll
  for (int i = 0; i < C::per_wave; ++i) {
    const int q = wave * C::per_wave + i, r = 8 * q + (lane >> 3);
    const int chunk = (lane & 7) ^ ((r >> 1) & 7);
    src[i] = (r < BM ? A + (size_t)min(row0 + r, a.M - 1) * a.lda
                     : W + (size_t)t_weight_row<EPI>(a, cb, r - BM) * a.ldw) + kbase + chunk * 8;
  }
  const int nk = a.kper / kTBK;
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
  if (gridDim.z > 1) {
    // split-K: the raw fp32 tile goes to this split's partial slice
    const int np = a.n_groups * kTBN;
    for (int i = tid; i < BM * kTBN / 4; i += C::threads) {
      const int r = i / (kTBN / 4), c4 = i % (kTBN / 4), row = row0 + r;
      if (row < a.M)
        *reinterpret_cast<float4 *>(a.part + ((size_t)kz * a.M + row) * np + cb * kTBN + 4 * c4) =
            *reinterpret_cast<const float4 *>(ct + r * kTCStride + 4 * c4);
    }
    return;
  }
  t_epilogue<EPI, BM, C::threads>(a, ct, rb, cb, layer, meta, true);
}

// Split-K reduction of a residual projection: X += p_0 + p_1 + ... (summed in
// split order, so deterministic), streamed as float4 over [M, N].
template <int S>
__global__ __launch_bounds__(256) void gemm_splitk_resid_kernel(const GemmArgs a) {
  const int n4 = a.N / 4;
  const size_t slice = (size_t)a.M * a.N;
  const int total = a.M * n4;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < total; i += gridDim.x * 256) {
    const int row = i / n4, c = 4 * (i - row * n4);
    float4 p[S];
#pragma unroll
    for (int z = 0; z < S; ++z) p[z] = *reinterpret_cast<const float4 *>(a.part + z * slice + (size_t)row * a.N + c);
    float4 *xp = reinterpret_cast<float4 *>(a.X + (size_t)row * a.ldx + c);
    float4 x = *xp;
    float4 v = p[0];
#pragma unroll
    for (int z = 1; z < S; ++z) {
      v.x += p[z].x;
      v.y += p[z].y;
      v.z += p[z].z;
      v.w += p[z].w;
    }
    x.x += v.x;
    x.y += v.y;
    x.z += v.z;
    x.w += v.w;
    *xp = x;
  }
}

// ---- 256 x 256 tiles, one 128 x 128 quadrant per wave ------------------------
//
// Four waves (one per SIMD) each accumulate a 128 x 128 quadrant as 4 x 4
// tiles of 32x32x16 products (256 fp32 accumulators per lane, held in the
// accumulation registers).  Per 16-deep k-substep a wave reads 8 fragments
// (8 KB) from LDS for 16 products, half the LDS reads and half the staged
// bytes per flop of the 64 x 64-per-wave kernel above.  A k-step is 32 deep.
//
// Staging (LDS-direct loads, all 160 KB of LDS):
//  * activations (A, 256 rows, L2-resident): a ring of 4 stages of one k-step,
//    64-byte rows (16 KB per stage);
//  * weights (W, 256 rows, streamed from HBM): a ring of 3 stages of two
//    k-steps, 128-byte rows (32 KB per stage), so that every weight request is
//    a whole 128-byte line -- 64-byte pieces of an 8 KB-stride matrix stream at
//    ~3.6 TB/s against ~6 TB/s for whole lines.
// Each step issues 4 loads of an activation stage 4 steps ahead and 4 loads
// (half) of a weight stage, so a wave always issues 8 per step and everything
// a step needs was issued at least 3 steps earlier.  With one wave per SIMD
// nothing else covers LDS latency, so each step's fragments are read during
// the previous step's products (two register sets); a buffer is refilled only
// after the barrier of the step following the one that read its fragments.
// Bank lines are 256 bytes: 64-byte rows XOR the 16-byte chunk index with
// (row / 4) mod 4, 128-byte rows with (row / 2) mod 8, so the 16 consecutive
// rows one quarter-wave reads land on 16 distinct bank groups.  The epilogue
// runs on one 128-column half at a time through the LDS tile, except the
// argmax, which each wave reduces from its own accumulators (its 128 columns
// are one 128-column block of the partials).
constexpr int kBT = 256, kBK = 32;

// (bv, bi) <- the larger of (bv, bi) and (ov, oi); equal values keep the lower
// column.  Values are never NaN here (a NaN never enters: see below), so this is
// a total order and any merge tree gives the same result as a scan in column
// order with a strict comparison.
__device__ __forceinline__ void amax_take(float &bv, int &bi, float ov, int oi) {
  const bool t = (ov > bv) | ((ov == bv) & (oi < bi));   // selects, no branch
  bv = t ? ov : bv;
  bi = t ? oi : bi;
}
// Value of the partner lane (lane ^ PX inside the 32 lanes of a half-wave):
// PX = 15, 7, 2, 1 by DPP lane moves inside 16-lane rows (row mirror, half-row
// mirror, quad permutations), PX = 16 through the LDS crossbar.
template <int PX> __device__ __forceinline__ int xchg(int x) {
  if constexpr (PX == 16) return __shfl_xor(x, 16);
  else if constexpr (PX == 15) return __builtin_amdgcn_mov_dpp(x, 0x140, 0xF, 0xF, false);
  else if constexpr (PX == 7) return __builtin_amdgcn_mov_dpp(x, 0x141, 0xF, 0xF, false);
  else if constexpr (PX == 2) return __builtin_amdgcn_mov_dpp(x, 0x4E, 0xF, 0xF, false);   // [2,3,0,1]
  else return __builtin_amdgcn_mov_dpp(x, 0xB1, 0xF, 0xF, false);                        // [1,0,3,2]
}
template <int PX> __device__ __forceinline__ float xchg(float x) {
  return __builtin_bit_cast(float, xchg<PX>(__builtin_bit_cast(int, x)));
}
// One exchange round over N row slots with the partner lane ^ PX: the lane
// whose bit HB is set keeps the upper half and hands the lower half over, its
// partner (bit HB clear) the reverse; each merges what it keeps with what it
// receives.  Partners must hold the same slots, so PX may flip only lane bits
// that no earlier round split on.
template <int N, int PX, int HB>
__device__ __forceinline__ void amax_round(float (&bv)[64], int (&bi)[64], int lane) {
  constexpr int H = N / 2;
  const bool hi = ((lane >> HB) & 1) != 0;
  float rv[H];
  int ri[H];
#pragma unroll
  for (int k = 0; k < H; ++k) {
    rv[k] = hi ? bv[k] : bv[k + H];
    ri[k] = hi ? bi[k] : bi[k + H];
  }
#pragma unroll
  for (int k = 0; k < H; ++k) {
    rv[k] = xchg<PX>(rv[k]);
    ri[k] = xchg<PX>(ri[k]);
  }
#pragma unroll
  for (int k = 0; k < H; ++k) {
    float kv = hi ? bv[k + H] : bv[k];
    int ki = hi ? bi[k + H] : bi[k];
    amax_take(kv, ki, rv[k], ri[k]);
    bv[k] = kv;
    bi[k] = ki;
  }
}
// Per-row (max, lowest column) of one wave's 128 x 128 quadrant, straight from
// its accumulators (rows row0 .., 128-column block blk of the argmax partials).
// Lane (fr, fk) holds columns 32j + fr of rows 32i + 8(e/4) + 4fk + e%4: it
// first scans its four columns of each of its 64 rows in column order (a NaN
// never wins; a row with no number above -inf keeps column 0), then five
// exchange rounds over the 32 lanes of its half-wave (partners lane ^ 15, ^ 7,
// ^ 2, ^ 1, ^ 16; upper halves kept by lanes with bit 3, 2, 1, 0, 4 set) leave
// it with row slots 2 * (16 b3 + 8 b2 + 4 b1 + 2 b0 + b4) + {0, 1} of the 64
// (b = bits of fr), reduced over all 128 columns.
__device__ __forceinline__ void quadrant_argmax(const GemmArgs &a, const f32x16 (&acc)[4][4], int row0, int blk,
                                                int lane) {
  const int fr = lane & 31, fk = lane >> 5;
  float bv[64];
  int bi[64];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float b = -INFINITY;
      int c = 0;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const bool t = acc[i][j][e] > b;
        b = t ? acc[i][j][e] : b;
        c = t ? 32 * j + fr : c;
      }
      bv[16 * i + e] = b;
      bi[16 * i + e] = c;
    }
  amax_round<64, 15, 3>(bv, bi, lane);
  amax_round<32, 7, 2>(bv, bi, lane);
  amax_round<16, 2, 1>(bv, bi, lane);
  amax_round<8, 1, 0>(bv, bi, lane);
  amax_round<4, 16, 4>(bv, bi, lane);
  const int s0 = 2 * (16 * ((fr >> 3) & 1) + 8 * ((fr >> 2) & 1) + 4 * ((fr >> 1) & 1) + 2 * (fr & 1) + (fr >> 4));
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int s = s0 + k, i = s >> 4, e = s & 15;
    const int row = row0 + 32 * i + 8 * (e >> 2) + 4 * fk + (e & 3);
    if (row < a.M) {
      a.amax_val[(size_t)row * a.n_groups + blk] = bv[k];
      a.amax_idx[(size_t)row * a.n_groups + blk] = blk * kTBN + bi[k];
    }
  }
}

constexpr int kBAStage = kBT * 64, kBAStages = 4;              // activation ring
constexpr int kBWStage = kBT * 128, kBWStages = 3;             // weight ring (two k-steps per stage)
constexpr int kBWBase = kBAStages * kBAStage;
constexpr int kBLdsStaging = kBWBase + kBWStages * kBWStage;   // 160 KB
constexpr int kBLds = kBLdsStaging > kBT * kTCStride * 4 ? kBLdsStaging : kBT * kTCStride * 4;
static_assert(kBLds >= kBT * kTCStride * 4 + kBT * 12, "epilogue row metadata fits past the fp32 tile");

template <int EPI>
__global__ __launch_bounds__(256) void gemm_big_kernel(const GemmArgs a, int n_rb, int n_ct, int per_xcd) {
  using T = bf16_t;
  __shared__ __align__(16) unsigned char lds[kBLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int layer = blockIdx.y;
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= n_rb * n_ct) return;
  const int ct_ = tile / n_rb, rb = tile % n_rb;
  const int n_cb = a.n_groups;                             // 128-column blocks
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const int row0 = rb * kBT;
  const RowMeta meta = load_row_meta<EPI, kBT>(a, row0, layer);

  // Activation piece i of a stage (this wave's 4 of 16): rows 16q .. 16q+15,
  // q = 4*wave + i; this lane fills row 16q + lane/4, 16-byte slot lane%4.
  // Weight piece i of half h of a stage (this wave's 4 of 16 per half): rows
  // 8q .. 8q+7, q = 16h + 4*wave + i; this lane fills row 8q + lane/8, slot
  // lane%8.  A second column block past the end re-reads the first (its
  // results are never stored).
  const T *asrc[4], *wsrc[2][4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * (4 * wave + i) + (lane >> 2);
    asrc[i] = A + (size_t)min(row0 + r, a.M - 1) * a.lda + ((lane & 3) ^ ((r >> 2) & 3)) * 8;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = 8 * (16 * h + 4 * wave + i) + (lane >> 3);
      int blk = 2 * ct_ + (c >> 7);
      if (blk >= n_cb) blk = 2 * ct_;
      wsrc[h][i] = W + (size_t)t_weight_row<EPI>(a, blk, c & 127) * a.ldw + ((lane & 7) ^ ((c >> 1) & 7)) * 8;
    }
  }
  const int nk = a.K / kBK, nw = nk / 2;
  const unsigned lds0 = lds_offset(lds);
  // activation stage s (one k-step) into ring slot s % 4; clamped past the end
  auto a_load = [&](int s, int i) {
    const int s_ = min(s, nk - 1);
    lds_dma16(asrc[i] + s_ * kBK, lds0 + (s % kBAStages) * kBAStage + (4 * wave + i) * 1024);
  };
  // half j % 2 of weight stage j / 2 (two k-steps) into ring slot (j / 2) % 3
  auto w_load = [&](int j, int i) {
    const int w = j >> 1, h = j & 1, w_ = min(w, nw - 1);
    lds_dma16(wsrc[h][i] + w_ * 2 * kBK, lds0 + kBWBase + (w % kBWStages) * kBWStage + (16 * h + 4 * wave + i) * 1024);
  };

  const int wr = wave >> 1, wc = wave & 1;
  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int fr = lane & 31, fk = lane >> 5;
  const int swa = (fr >> 2) & 3, sww = (fr >> 1) & 7;      // swizzles of this lane's fragment rows
  // Fragment g of step kt (g = 4 * substep + i): A rows wr*128 + 32i .. of
  // activation slot kt % 4, W rows wc*128 + 32i .. of weight slot (kt/2) % 3,
  // whose 128-byte rows hold step kt in chunks 4*(kt%2) .. +3.
  auto read_frag = [&](int kt, int g, Frag<T> (&af)[2][4], Frag<T> (&bf)[2][4]) {
    const int sub = g >> 2, i = g & 3, c = 2 * sub + fk;
    const unsigned char *ab = lds + (kt % kBAStages) * kBAStage;
    const unsigned char *wb = lds + kBWBase + ((kt >> 1) % kBWStages) * kBWStage;
    af[sub][i].v = *reinterpret_cast<const uint4 *>(ab + (wr * 128 + i * 32 + fr) * 64 + ((c ^ swa) << 4));
    bf[sub][i].v = *reinterpret_cast<const uint4 *>(wb + (wc * 128 + i * 32 + fr) * 128 + (((4 * (kt & 1) + c) ^ sww) << 4));
  };
  // Step kt: wait until only the loads of steps kt-2 and kt-1 are outstanding
  // (everything step kt+1 needs was issued by step kt-3), barrier; then 8
  // groups of 4 products on the fragments of step kt (read during step kt-1),
  // each followed by one load -- activation stage kt+4 into the slot of stage
  // kt (read during step kt-1), then half kt+5 of the weight ring (its slot
  // was last read during step kt-1 or kt-2) -- and two fragment reads of step
  // kt+1.  Spreading the loads between the products keeps the memory and LDS
  // queues from holding up the matrix cores; the scheduling barriers pin the
  // order.  lgkmcnt field cleared: the wait also covers this wave's fragment
  // reads of the previous step (long done), so the compiler adds no wait of
  // its own.
  constexpr int kLgkm0 = ~(0xF << 8);
#define DF_BSTEP(kt, FA, FB, GA, GB)                                                                \
  do {                                                                                              \
    asm volatile("" ::: "memory");                                                                  \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(16) & kLgkm0);                                             \
    __builtin_amdgcn_s_barrier();                                                                   \
    asm volatile("" ::: "memory");                                                                  \
    _Pragma("unroll") for (int g = 0; g < 8; ++g) {                                                 \
      const int sub_ = g >> 2, i_ = g & 3;                                                          \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) acc[i_][j] = mma32(acc[i_][j], FA[sub_][i_], FB[sub_][j]); \
      if (g < 4) a_load((kt) + 4, g);                                                               \
      else w_load((kt) + 5, g - 4);                                                                 \
      read_frag((kt) + 1, g, GA, GB);                                                               \
      __builtin_amdgcn_sched_barrier(0);                                                            \
    }                                                                                               \
  } while (0)
  Frag<T> a0[2][4], b0[2][4], a1[2][4], b1[2][4];
  // prologue, in the steady state's order: weight half 0, then for p = -4 .. -1
  // activation stage p+4 and weight half p+5
#pragma unroll
  for (int i = 0; i < 4; ++i) w_load(0, i);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a_load(p, i);
#pragma unroll
    for (int i = 0; i < 4; ++i) w_load(p + 1, i);
  }
  // step 0's activation stage and both weight halves were issued before the
  // last three rounds of 8
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(24));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int g = 0; g < 8; ++g) read_frag(0, g, a0, b0);
  // nk is even (K is a multiple of 64)
  for (int kt = 0; kt < nk; kt += 2) {
    DF_BSTEP(kt, a0, b0, a1, b1);
    DF_BSTEP(kt + 1, a1, b1, a0, b0);
  }
#undef DF_BSTEP
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  if constexpr (EPI == EPI_ARGMAX) {
    // a wave's 128 columns are exactly one 128-column block of the partials
    const int blk = 2 * ct_ + wc;
    if (blk < n_cb) quadrant_argmax(a, acc, row0 + wr * 128, blk, lane);
    return;
  }
  float *ctile = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int blk = 2 * ct_ + h;
    if (blk >= n_cb) break;
    if (wc == h) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e)
            ctile[(wr * 128 + i * 32 + 8 * (e / 4) + 4 * fk + e % 4) * kTCStride + j * 32 + fr] = acc[i][j][e];
    }
    __syncthreads();
    t_epilogue<EPI, kBT, 256>(a, ctile, rb, blk, layer, meta, h == 0);
    __syncthreads();
  }
}

// ---- 256 x 192 tiles for gate/up + SwiGLU -------------------------------------
//
// The 256 x 256 kernel's schedule with 192 weight rows per tile (96 gate rows
// beside their 96 up rows): each wave accumulates 128 rows x 96 columns as
// 4 x 3 tiles of 32x32x16 products, so a 512-row gate/up of FFN 12288 is 256
// tiles, one per compute unit, instead of 192 tiles of 256 x 256 that leave a
// quarter of the compute units idle.  Per step a wave issues 4 activation and
// 3 weight loads (weight stage: 192 rows of 128 bytes, 24 pieces of 1 KB, half
// a stage per step).  The smaller weight stages leave room for a fourth one,
// so weight halves are requested 7 steps ahead instead of 5 (the weights come
// from HBM; the loop waits on them, not on the matrix cores).  K is walked in the same order as the 256 x 256 kernel,
// so both give identical sums.  Epilogue: gate and up values pass through LDS
// one 128-row half at a time, and all four waves write silu(gate) * up in
// 16-byte pieces.
constexpr int kB3N = 192, kB3WStage = kB3N * 128, kB3WStages = 4;
constexpr int kB3WBase = kBAStages * kBAStage;
constexpr int kB3Lds = kB3WBase + kB3WStages * kB3WStage;   // 160 KB
constexpr int kB3Row = 100;                                  // floats per epilogue row (96 + 4)
static_assert(2 * 128 * kB3Row * 4 <= kB3Lds, "gate and up values of 128 rows fit");

__global__ __launch_bounds__(256) void gemm_swiglu192_kernel(const GemmArgs a, int n_rb, int n_ct, int per_xcd) {
  using T = bf16_t;
  constexpr int NJ = 3, WPW = 3;                           // column tiles and weight loads per wave
  __shared__ __align__(16) unsigned char lds[kB3Lds];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int layer = blockIdx.y;
  // row-block-major order: an XCD's tiles share one 256-row block of the
  // activations (2 MB at 4096 columns, resident in that XCD's L2 beside the
  // weight stream) instead of needing both
  const int tile = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (tile >= n_rb * n_ct) return;
  const int rb = tile / n_ct, ct_ = tile % n_ct;
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const int row0 = rb * kBT;

  // activation pieces as in the 256 x 256 kernel; weight piece i of half h:
  // rows 8q .. 8q+7, q = 12h + 3*wave + i (tile column c -> gate row ct*96 + c
  // for c < 96, else up row ffn + ct*96 + c - 96)
  const T *asrc[4], *wsrc[2][WPW];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int r = 16 * (4 * wave + i) + (lane >> 2);
    asrc[i] = A + (size_t)min(row0 + r, a.M - 1) * a.lda + ((lane & 3) ^ ((r >> 2) & 3)) * 8;
  }
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int c = 8 * (12 * h + WPW * wave + i) + (lane >> 3);
      const int wrow = c < 96 ? ct_ * 96 + c : a.ffn + ct_ * 96 + (c - 96);
      wsrc[h][i] = W + (size_t)wrow * a.ldw + ((lane & 7) ^ ((c >> 1) & 7)) * 8;
    }
  const int nk = a.K / kBK, nw = nk / 2;
  const unsigned lds0 = lds_offset(lds);
  auto a_load = [&](int s, int i) {
    const int s_ = min(s, nk - 1);
    lds_dma16(asrc[i] + s_ * kBK, lds0 + (s % kBAStages) * kBAStage + (4 * wave + i) * 1024);
  };
  auto w_load = [&](int j, int i) {
    const int w = j >> 1, h = j & 1, w_ = min(w, nw - 1);
    lds_dma16(wsrc[h][i] + w_ * 2 * kBK,
              lds0 + kB3WBase + (w % kB3WStages) * kB3WStage + (12 * h + WPW * wave + i) * 1024);
  };

  const int wr = wave >> 1, wc = wave & 1;
  f32x16 acc[4][NJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  const int fr = lane & 31, fk = lane >> 5;
  const int swa = (fr >> 2) & 3, sww = (fr >> 1) & 7;
  auto read_frag = [&](int kt, int g, Frag<T> (&af)[2][4], Frag<T> (&bf)[2][NJ]) {
    const int sub = g >> 2, i = g & 3, c = 2 * sub + fk;
    const unsigned char *ab = lds + (kt % kBAStages) * kBAStage;
    const unsigned char *wb = lds + kB3WBase + ((kt >> 1) % kB3WStages) * kB3WStage;
    af[sub][i].v = *reinterpret_cast<const uint4 *>(ab + (wr * 128 + i * 32 + fr) * 64 + ((c ^ swa) << 4));
    if (i < NJ)
      bf[sub][i].v = *reinterpret_cast<const uint4 *>(wb + (wc * 96 + i * 32 + fr) * 128 +
                                                      (((4 * (kt & 1) + c) ^ sww) << 4));
  };
  constexpr int kLgkm0 = ~(0xF << 8);
  constexpr int kPerStep = 4 + WPW;                        // loads a wave issues per step
#define DF_B3STEP(kt, FA, FB, GA, GB)                                                               \
  do {                                                                                              \
    asm volatile("" ::: "memory");                                                                  \
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(2 * kPerStep) & kLgkm0);                                   \
    __builtin_amdgcn_s_barrier();                                                                   \
    asm volatile("" ::: "memory");                                                                  \
    _Pragma("unroll") for (int g = 0; g < 8; ++g) {                                                 \
      const int sub_ = g >> 2, i_ = g & 3;                                                          \
      _Pragma("unroll") for (int j = 0; j < NJ; ++j) acc[i_][j] = mma32(acc[i_][j], FA[sub_][i_], FB[sub_][j]); \
      if (g < 4) a_load((kt) + 4, g);                                                               \
      else if (g - 4 < WPW) w_load((kt) + 7, g - 4);                                                \
      read_frag((kt) + 1, g, GA, GB);                                                               \
      __builtin_amdgcn_sched_barrier(0);                                                            \
    }                                                                                               \
  } while (0)
  // prologue in the steady state's order: weight halves 0..2, then for
  // p = -4 .. -1 activation stage p+4 and weight half p+7.  Step kt waits for
  // everything issued before step kt-2; a weight half issued at step kt lands
  // in the slot of a stage whose last fragments were read during step kt-1.
  Frag<T> a0[2][4], b0[2][NJ], a1[2][4], b1[2][NJ];
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int i = 0; i < WPW; ++i) w_load(j, i);
#pragma unroll
  for (int p = 0; p < 4; ++p) {
#pragma unroll
    for (int i = 0; i < 4; ++i) a_load(p, i);
#pragma unroll
    for (int i = 0; i < WPW; ++i) w_load(p + 3, i);
  }
  // step 0 needs weight halves 0, 1 and activation stage 0: all but the last
  // 3 rounds of 7 and the 3 loads of half 3
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(3 * kPerStep + WPW));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int g = 0; g < 8; ++g) read_frag(0, g, a0, b0);
  for (int kt = 0; kt < nk; kt += 2) {
    DF_B3STEP(kt, a0, b0, a1, b1);
    DF_B3STEP(kt + 1, a1, b1, a0, b0);
  }
#undef DF_B3STEP
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");

  // Two passes over the row halves: in pass p the two waves with wr == p put
  // their gate (wc = 0) and up (wc = 1) values in LDS ([128 rows][kB3Row]
  // fp32 each), then all four waves write silu(gate) * up for those 128 rows,
  // 8 columns (16 bytes) per store.
  float *gl = reinterpret_cast<float *>(lds), *ul = gl + 128 * kB3Row;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    if (wr == p) {
      float *dst = wc ? ul : gl;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
          for (int e = 0; e < 16; ++e) dst[(i * 32 + 8 * (e / 4) + 4 * fk + e % 4) * kB3Row + j * 32 + fr] = acc[i][j][e];
    }
    __syncthreads();
    for (int q = tid; q < 128 * 12; q += 256) {
      const int rl = q / 12, c8 = (q % 12) * 8, row = row0 + p * 128 + rl;
      if (row < a.M) {
        const float4 g0 = *reinterpret_cast<const float4 *>(gl + rl * kB3Row + c8);
        const float4 g1 = *reinterpret_cast<const float4 *>(gl + rl * kB3Row + c8 + 4);
        const float4 u0 = *reinterpret_cast<const float4 *>(ul + rl * kB3Row + c8);
        const float4 u1 = *reinterpret_cast<const float4 *>(ul + rl * kB3Row + c8 + 4);
        const float f[8] = {silu_mul(g0.x, u0.x), silu_mul(g0.y, u0.y), silu_mul(g0.z, u0.z), silu_mul(g0.w, u0.w),
                            silu_mul(g1.x, u1.x), silu_mul(g1.y, u1.y), silu_mul(g1.z, u1.z), silu_mul(g1.w, u1.w)};
        Frag<T> o;
        o.set(f);
        o.store((T *)a.out + (size_t)row * a.ldo + ct_ * 96 + c8);
      }
    }
    __syncthreads();
  }
}

template <int EPI>
static void launch_big_t(const GemmArgs &a, int z_slices, hipStream_t st) {
  const int n_rb = (a.M + kBT - 1) / kBT, n_ct = (a.n_groups + 1) / 2;
  const int per_xcd = (n_rb * n_ct + 7) / 8;
  hipLaunchKernelGGL((gemm_big_kernel<EPI>), dim3(8 * per_xcd, z_slices), dim3(256), 0, st, a, n_rb, n_ct, per_xcd);
}

static hipError_t launch_big(Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  switch (epi) {
    case EPI_STORE: launch_big_t<EPI_STORE>(a, z_slices, st); break;
    case EPI_STORE_F32: launch_big_t<EPI_STORE_F32>(a, z_slices, st); break;
    case EPI_RESID: launch_big_t<EPI_RESID>(a, z_slices, st); break;
    case EPI_SWIGLU: launch_big_t<EPI_SWIGLU>(a, z_slices, st); break;
    case EPI_QKV: launch_big_t<EPI_QKV>(a, z_slices, st); break;
    case EPI_INJECT: launch_big_t<EPI_INJECT>(a, z_slices, st); break;
    case EPI_ARGMAX: launch_big_t<EPI_ARGMAX>(a, z_slices, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int gemm_tiled_cols(Epilogue epi, int N, int ffn) { return epi == EPI_SWIGLU ? ffn / 64 : N / kTBN; }

bool gemm_tiled_ok(Epilogue epi, int N, int K, int ffn, int hd) {
  if (K % kTBK) return false;
  if (epi == EPI_SWIGLU) return ffn % 64 == 0;
  if ((epi == EPI_QKV || epi == EPI_INJECT) && (kTBN % hd || hd % 16)) return false;   // 8-pair groups
  return N % kTBN == 0;
}

template <int BM>
static hipError_t launch_tiled_bm(Epilogue epi, const GemmArgs &a, int z_slices, int splits, hipStream_t st) {
  const int n_rb = (a.M + BM - 1) / BM;
  const int n_cb = a.n_groups;
  const int per_xcd = (n_rb * n_cb + 7) / 8;
  dim3 grid(8 * per_xcd, z_slices, splits), block(TCfg<BM>::threads);
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

static void launch_splitk_resid(const GemmArgs &a, int splits, int cu, hipStream_t st) {
  const long f4 = (long)a.M * (a.N / 4);
  const int grid = (int)std::min<long>((f4 + 255) / 256, 8L * cu);
  if (splits == 2) hipLaunchKernelGGL((gemm_splitk_resid_kernel<2>), dim3(grid), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((gemm_splitk_resid_kernel<4>), dim3(grid), dim3(256), 0, st, a);
}

// 256 x 256 tiles when they number at least kBigMinTiles; otherwise 256 x 128
// tiles when those give a few workgroups per compute unit, else 128 x 128.
// A 128 x 128 launch that leaves compute units idle splits K over 2 or 4
// workgroups per tile (when a partial buffer is given and each split keeps at
// least 1024 of K; residual epilogue only): the splits write fp32 partial
// tiles and a streaming kernel adds their sum to the residual.
hipError_t launch_gemm_tiled(Epilogue epi, GemmArgs &a, int z_slices, int cu, hipStream_t st) {
  a.kper = a.K;
  const long big_tiles = (long)((a.M + kBT - 1) / kBT) * ((a.n_groups + 1) / 2) * z_slices;
  if (a.M > 128 && big_tiles >= kBigMinTiles) {
    // gate/up: 256 x 192 tiles where they fill the compute units' rounds
    // better than 256 x 256 (e.g. 512 rows of FFN 12288: 256 tiles against 192);
    // its epilogue stores 8 outputs (16 bytes) at a time
    if (epi == EPI_SWIGLU && a.ffn % 96 == 0 && a.K % (2 * kBK) == 0 && a.ldo % 8 == 0 &&
        reinterpret_cast<uintptr_t>(a.out) % 16 == 0) {
      const int n_rb = (a.M + kBT - 1) / kBT, n_ct3 = a.ffn / 96;
      const long t3 = (long)n_rb * n_ct3 * z_slices;
      const double fill3 = (double)t3 / (double)(((t3 + cu - 1) / cu) * cu);
      const double fill4 = (double)big_tiles / (double)(((big_tiles + cu - 1) / cu) * cu);
      if (fill3 > fill4 * 1.05) {
        const int per_xcd = (int)((n_rb * (long)n_ct3 + 7) / 8);
        hipLaunchKernelGGL(gemm_swiglu192_kernel, dim3(8 * per_xcd, z_slices), dim3(256), 0, st, a, n_rb, n_ct3,
                           per_xcd);
        return hipGetLastError();
      }
    }
    return launch_big(epi, a, z_slices, st);
  }
  // 256 x 128 tiles (half the staged bytes per flop of 128 x 128) when their
  // rounds of the compute units take no longer, counted in 128 x 128 tiles
  // (e.g. 2048 x 4096: 256 tiles, one round, against 512 in two)
  const long tiles256 = (long)((a.M + 255) / 256) * a.n_groups * z_slices;
  const long tiles = (long)((a.M + 127) / 128) * a.n_groups * z_slices;
  if (tiles256 >= cu && 2 * ((tiles256 + cu - 1) / cu) <= (tiles + cu - 1) / cu)
    return launch_tiled_bm<256>(epi, a, z_slices, 1, st);
  // residual projection with a long K (the batched down projection, 512 rows
  // of K = 12288): 256 x 128 tiles split over K fill the compute units with
  // half the staged bytes per flop of 128 x 128 ones, when each split keeps at
  // least 2048 of K (down 79.8 -> 71.9 us with the reduction; the O
  // projection's 1024-long splits measured slower and keep 128 x 128)
  if (a.part && z_slices == 1 && epi == EPI_RESID && a.M > 128) {
    int s2 = 1;
    while (s2 < 4 && tiles256 * s2 < cu && a.K % (s2 * 2 * kTBK) == 0 && a.K / (s2 * 2) >= 2048 &&
           (size_t)s2 * 2 * a.M * a.n_groups * kTBN * 4 <= a.part_bytes)
      s2 *= 2;
    if (s2 > 1 && tiles256 * s2 >= cu) {
      a.kper = a.K / s2;
      hipError_t e = launch_tiled_bm<256>(epi, a, z_slices, s2, st);
      if (e != hipSuccess) return e;
      launch_splitk_resid(a, s2, cu, st);
      return hipGetLastError();
    }
  }
  int splits = 1;
  if (a.part && z_slices == 1 && epi == EPI_RESID) {
    while (splits < 4 && tiles * splits * 2 <= cu && a.K % (splits * 2 * kTBK) == 0 && a.K / (splits * 2) >= 1024 &&
           (size_t)splits * 2 * a.M * a.n_groups * kTBN * 4 <= a.part_bytes)
      splits *= 2;
  }
  a.kper = a.K / splits;
  hipError_t e = launch_tiled_bm<128>(epi, a, z_slices, splits, st);
  if (e != hipSuccess || splits == 1) return e;
  launch_splitk_resid(a, splits, cu, st);
  return hipGetLastError();
}

}  // namespace dflash
