// Persistent weight-streaming GEMM for up to 16 activation rows: the batch-1
// (and small-batch) projections of the drafter step, bound by HBM bandwidth.
//
// out[M, N] = A[M, K] * W[N, K]^T with M <= 16, W row-major [out, in].
//
// One 16-wave workgroup runs per compute unit and walks 16-column tiles
// round-robin (tile = block, block + grid, ...).  For every tile the 16 waves
// split the k-chunk steps evenly and their partial tiles are summed through LDS
// in wave order; the next tile's weight fragments are already in flight while
// a tile is reduced and its epilogue runs, so the HBM stream does not stop
// between tiles.  bf16 weights are read in whole 128-byte lines with the
// non-temporal hint (see StreamBuf).
//
// The activation rows are staged in LDS once per workgroup when all of K fits
// (K <= 4096 in bf16): as a copy, or as RMSNorm(X) * gain computed from the fp32
// residual stream (optionally gathered from the embedding first).  Longer K
// (the down projection, the context-fusion projection) reads the activation
// fragments straight from global memory, prefetched with the weights.
//
// Column maps and epilogues are those of the few-rows GEMM (RoPE pairs, SwiGLU
// pairs, residual add, storage, per-row argmax).
//
// Tile width TW = 8 (bf16 QKV with resident rows): a tile is 4 RoPE pairs (8
// weight rows), so that 6144 QKV columns make 768 tiles, 3 per workgroup on all
// 256 compute units, where 384 16-column tiles leave a quarter of them idle.
// TW = 32 (bf16 down projection, K past the resident capacity): a pair of
// workgroups shares a 32-column tile, each over half of K, so a compute unit
// reads half the activation fragments for the same weight bytes (down
// 29.1 -> 25.4 us per layer, Qwen3-8B shape); the pair's second workgroup to
// finish adds the two halves to the residual.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kSWaves = 16;
constexpr int kSThreads = kSWaves * 64;
constexpr int kSResBytes = 128 * 1024;   // LDS budget of the resident activation rows

enum AMode { A_GLOBAL = 0, A_COPY = 1, A_NORM = 2, A_EMBED_NORM = 3, A_COPY_ROWS = 6, A_TW8 = 16, A_SPLIT2 = 32 };

// the QKV epilogues (with or without the copy into the paged cache)
constexpr bool qkv_epi(int e) { return e == EPI_QKV || e == EPI_QKV_CACHE; }

template <typename T>
__host__ __device__ constexpr int stream_res_k() {
  return kSResBytes / (16 * (int)sizeof(T));
}

// weight row of column c (0 .. TW-1) of tile t
template <int EPI, int TW = 16>
__device__ __forceinline__ int s_weight_row(const GemmArgs &a, int t, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    return c < 8 ? t * 8 + c : a.ffn + t * 8 + (c - 8);
  } else if constexpr (qkv_epi(EPI) || EPI == EPI_INJECT) {
    constexpr int P = TW / 2;                      // RoPE pairs per tile
    const int tph = a.hd / TW;
    const int h = t / tph, j0 = (t - h * tph) * P;
    return h * a.hd + (c < P ? j0 + c : a.hd / 2 + j0 + (c - P));
  } else {
    return t * TW + c;
  }
}

// Epilogue operands that do not depend on the weights, read at kernel start so
// that the epilogue issues no dependent global load: the residual element of
// the workgroup's first tile (thread tid < 256 owns row tid / 16, column
// tid % 16) and the context length of the thread's row (QKV, tid < 16 * TW / 2).
// Indices are clamped so every thread loads from a valid address.
struct EpiPre {
  float x;
  int ctx;
  int page;   // QKV with a cache copy: page of the thread's row position (read after the staging loads)
};

template <int EPI, int TW>
__device__ __forceinline__ EpiPre s_epi_pre(const GemmArgs &a, int t0) {
  EpiPre p{0.f, 0, 0};
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_RESID && TW == 32) {
    // split pair: thread tid < 512 owns row (tid / 16) % 16, column
    // 16 (tid / 256) + tid % 16 of the 32-column tile
    const int r = min((tid >> 4) & 15, a.M - 1), c = 16 * ((tid >> 8) & 1) + (tid & 15);
    p.x = a.X[(size_t)r * a.ldx + t0 * 32 + c];
  } else if constexpr (EPI == EPI_RESID) {
    const int r = min(tid >> 4, a.M - 1), c = tid & 15;
    p.x = a.X[(size_t)r * a.ldx + t0 * 16 + c];
  } else if constexpr (qkv_epi(EPI)) {
    p.ctx = a.ctx_len[min(tid / (TW / 2), a.M - 1) / a.block_size];
  }
  return p;
}

// Epilogue of one 16 x 16 tile held in LDS (ct, row-major [16][16], columns
// 0 .. TW-1 valid); ``first`` marks the workgroup's first tile, whose residual
// elements are in ``pre``.
template <typename T, int EPI, int TW>
__device__ __forceinline__ void s_epilogue(const GemmArgs &a, const float *ct, int t, int layer, float *best_v,
                                           int *best_i, const double *inv_freq, const EpiPre &pre, bool first) {
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    if (tid < 256) {
      const int r = tid >> 4, c = tid & 15;
      if (r < a.M) {
        const int n = t * 16 + c;
        const float v = ct[tid];
        if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)r * a.ldo + n, v);
        else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)r * a.ldo + n] = v;
        else {
          // two separate paths: merged, the wait for the later-tile load would
          // also stall the first tile (and drain the weights in flight)
          float *xp = a.X + (size_t)r * a.ldx + n;
          float nv;
          if (first) {
            nv = pre.x + v;
            asm volatile("; residual from prefetch" : "+v"(nv));
          } else {
            nv = *xp + v;
            asm volatile("; residual loaded" : "+v"(nv));
          }
          *xp = nv;
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    if (tid < 128) {
      const int r = tid >> 3, c = tid & 7;
      if (r < a.M) {
        const float gt = ct[r * 16 + c], up = ct[r * 16 + 8 + c];
        Storage<T>::store((T *)a.out, (size_t)r * a.ldo + t * 8 + c, silu_mul(gt, up));
      }
    }
  } else if constexpr (qkv_epi(EPI) || EPI == EPI_INJECT) {
    constexpr int P = TW / 2;                         // RoPE pairs per tile
    if (tid < 16 * P) {
      const int r = tid / P, c = tid % P;
      if (r < a.M) {
        const int hd = a.hd, half = hd / 2;
        const int nqh = (qkv_epi(EPI)) ? a.nq : 0;  // q heads in the output
        const int qcols = nqh * hd;
        const int kcols = a.nkv * hd;
        const int h = t / (hd / TW);                  // head of this tile (uniform)
        const int j0 = (t % (hd / TW)) * P;
        const int n = s_weight_row<EPI, TW>(a, t, c);
        const float x1 = ct[r * 16 + c], x2 = ct[r * 16 + P + c];
        int pos;
        size_t slot = 0;
        if constexpr (qkv_epi(EPI)) {
          pos = pre.ctx + r % a.block_size;
        } else {
          pos = a.pos[r];
          const int s = a.seq[r];
          const int page = a.block_table[(size_t)s * a.max_pages + pos / a.page_size];
          slot = (size_t)layer * a.cache_layer_stride + ((size_t)page * a.page_size + (pos % a.page_size)) * kcols;
        }
        float lo = x1, hi = x2;
        if (h < nqh + a.nkv) {                        // q and k heads rotate
          float cs, sn;
          rope_cs_inv(pos, inv_freq[j0 + c], &cs, &sn);
          lo = x1 * cs - x2 * sn;
          hi = x2 * cs + x1 * sn;
        }
        // the destination depends on the head only, so it is chosen per tile
        T *dst;
        size_t off;
        if (h < nqh) {
          dst = (T *)a.q_out;
          off = (size_t)r * qcols + n;
        } else if (h < nqh + a.nkv) {
          dst = (T *)a.k_out;
          off = (qkv_epi(EPI) ? (size_t)r * kcols : slot) + (n - qcols);
        } else {
          dst = (T *)a.v_out;
          off = (qkv_epi(EPI) ? (size_t)r * kcols : slot) + (n - qcols - kcols);
        }
        Storage<T>::store(dst, off, lo);
        Storage<T>::store(dst, off + half, hi);
        if constexpr (EPI == EPI_QKV_CACHE) {
          if (h >= nqh) {   // target verify: the block's k, v also join the cache
            const int pos = pre.ctx + r % a.block_size;
            const size_t cs = ((size_t)pre.page * a.page_size + pos % a.page_size) * kcols +
                              (h < nqh + a.nkv ? n - qcols : n - qcols - kcols);
            T *cdst = (T *)(h < nqh + a.nkv ? a.kc_out : a.vc_out);
            Storage<T>::store(cdst, cs, lo);
            Storage<T>::store(cdst, cs + half, hi);
          }
        }
      }
    }
  } else if constexpr (EPI == EPI_ARGMAX) {
    // running (max, lowest id) per row across this workgroup's tiles; tiles
    // arrive in increasing order, so a strict comparison keeps the lowest id.
    // A NaN never compares greater, so it never wins; the first tile always
    // sets the id (best_i < 0), which keeps it a valid column when a row holds
    // no number above -inf.
    if (tid < 16) {
      float b = -INFINITY;
      int bc = 0;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float v = ct[tid * 16 + c];
        if (v > b) { b = v; bc = c; }
      }
      if (b > *best_v || *best_i < 0) { *best_v = b; *best_i = t * 16 + bc; }
    }
  }
}

// One batch of weight fragments (and, when the activations are not resident,
// activation fragments) for one lane: U 1 KB loads per wave.
//
// bf16: every weight load covers whole 128-byte lines, 8 weight rows at two
// consecutive 32-wide k-chunks (a chunk step of 64): lane (l % 16, l / 16)
// reads row r0 + (l % 8) at chunk 2c + (l % 16) / 8, bytes 16 (l / 16) ..  A
// 16-column tile takes two such loads per step (rows 0-7, rows 8-15), an
// 8-column tile one.  Two products per load, with the activation fragments of
// chunk 2c and of chunk 2c + 1, leave the even chunk's dot products in columns
// 0-7 of one accumulator and the odd chunk's in columns 8-15 of another (fold
// combines them).  Streamed reads of whole lines with the non-temporal hint
// measured 6.7 TB/s, half lines 5.6-5.9 TB/s (plain or non-temporal), so the
// weights take this layout and the hint.  The QKV projection alone keeps plain
// loads: with the hint the block attention launched after it ran 1.2 us
// longer per layer, while QKV itself gained 0.2 us (measured, batch 1).
// fp32: a 32-wide chunk of a row is already a whole line; one plain load per
// chunk step.
//
// Loads are issued unconditionally: a step past the wave's range reads the
// last valid step of the row instead, and its product is masked to zero at
// compute time.  Branch-free issue lets the compiler count outstanding loads
// exactly, so consuming one buffer waits only for that buffer's loads while
// the other buffer's batch stays in flight.  Lanes of rows >= M read row 0;
// their output rows are never stored.
template <typename T, int U, bool RES, int TW = 16>
struct StreamBuf {
  static constexpr bool WL = sizeof(T) == 2;           // whole-line layout (bf16)
  static_assert(TW == 16 || WL, "8- and 32-column tiles: bf16");
  static constexpr int NR = WL ? TW / 8 : 1;           // loads per chunk step
  static constexpr int S = U / NR;                     // chunk steps per batch
  static constexpr int CE = WL ? 64 : 32;              // k-elements per chunk step
  static constexpr int NA = WL ? 2 * NR : 1;           // accumulators
  static_assert(S * NR == U, "whole steps per batch");
  Frag<T> w[U];                                        // step j, row group r: w[NR * j + r]
  Frag<T> x[RES ? 1 : (WL ? 2 : 1) * S];

  // arow: the lane's activation pointer (resident rows: in LDS; bf16 from
  // global memory: rows 0-7 in the whole-line layout, arow_hi rows 8-15)
  template <int EPI>
  __device__ __forceinline__ void issue(const GemmArgs &a, const T *W, const T *arow, const T *arow_hi, int t, int c0,
                                        int clast) {
    const int ln = threadIdx.x & 15, g = (threadIdx.x >> 4) & 3;
    const T *wp[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r)
      wp[r] = WL ? W + (size_t)s_weight_row<EPI, TW>(a, t, 8 * r + (ln & 7)) * a.ldw + 8 * g + 32 * (ln >> 3)
                 : W + (size_t)s_weight_row<EPI, TW>(a, t, ln) * a.ldw + 8 * g;
    __builtin_amdgcn_sched_barrier(0);   // loads issued before the batch stay before it
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const int c = min(c0 + j, clast);
#pragma unroll
      for (int r = 0; r < NR; ++r) {
        if constexpr (WL && !qkv_epi(EPI)) w[NR * j + r].load_stream(wp[r] + CE * c);
        else w[NR * j + r].load(wp[r] + CE * c);
      }
      if constexpr (!RES) {
        if constexpr (WL) {
          x[2 * j].load(arow + 64 * c);
          x[2 * j + 1].load(arow_hi + 64 * c);
        } else {
          x[j].load(arow + 32 * c);
        }
      }
    }
    // the scheduler would otherwise sink the loads below the products that
    // free their registers, which serialises the stream
    __builtin_amdgcn_sched_barrier(0);
  }

  __device__ __forceinline__ void compute(f32x4 (&acc)[NA], const T *arow, int c0, int cend, int clast) const {
#pragma unroll
    for (int j = 0; j < S; ++j) {
      const bool on = c0 + j < cend;
      const int c = min(c0 + j, clast);
      if constexpr (WL) {
        Frag<T> a0, a1;
        if constexpr (RES) {
          a0.load(arow + 64 * c);
          a1.load(arow + 64 * c + 32);
        } else {
          // whole-line activation loads back to the product layout.  x[2j]
          // holds rows 0-7 (lane l % 16 < 8: row l % 16, chunk 2c; lane
          // l % 16 >= 8: row l % 16 - 8, chunk 2c + 1), x[2j + 1] rows 8-15 the
          // same way.  A lane of row r < 8 keeps its chunk-2c piece and takes
          // the chunk-2c+1 piece from lane l ^ 8; a lane of row r >= 8 keeps
          // its chunk-2c+1 piece and takes the chunk-2c piece from lane l ^ 8.
          const bool lo = (threadIdx.x & 15) < 8;
          const Frag<T> sa = xor8(x[2 * j]), sb = xor8(x[2 * j + 1]);
          a0 = lo ? x[2 * j] : sb;
          a1 = lo ? sa : x[2 * j + 1];
        }
#pragma unroll
        for (int r = 0; r < NR; ++r) {
          Frag<T> wj = w[NR * j + r];
          if (!on) wj.zero();
          acc[2 * r] = mma(acc[2 * r], a0, wj);
          acc[2 * r + 1] = mma(acc[2 * r + 1], a1, wj);
        }
      } else {
        Frag<T> wj = w[j], af;
        if (!on) wj.zero();
        if constexpr (RES) af.load(arow + 32 * c); else af = x[j];
        acc[0] = mma(acc[0], af, wj);
      }
    }
  }

  // the fragment of lane l ^ 8 (a 16-lane row rotated by 8)
  __device__ __forceinline__ static Frag<T> xor8(const Frag<T> &f) {
    Frag<T> o;
    if constexpr (sizeof(T) == 2) {
      o.v.x = __builtin_amdgcn_mov_dpp((int)f.v.x, 0x128, 0xF, 0xF, false);
      o.v.y = __builtin_amdgcn_mov_dpp((int)f.v.y, 0x128, 0xF, 0xF, false);
      o.v.z = __builtin_amdgcn_mov_dpp((int)f.v.z, 0x128, 0xF, 0xF, false);
      o.v.w = __builtin_amdgcn_mov_dpp((int)f.v.w, 0x128, 0xF, 0xF, false);
    } else {
      o = f;
    }
    return o;
  }

  // the tile's 16 x 16 result in the fragment layout of one product (lane:
  // column l % 16), the accumulators cleared
  __device__ __forceinline__ static f32x4 fold(f32x4 (&acc)[NA]) {
    f32x4 o;
    if constexpr (!WL) {
      o = acc[0];
    } else if constexpr (NR == 1) {
#pragma unroll
      for (int i = 0; i < 4; ++i) o[i] = acc[0][i] + __shfl_xor(acc[1][i], 8);
    } else {
      // columns 0-7: rows 0-7 (acc 0 even, acc 1 odd chunks from lane l ^ 8);
      // columns 8-15: rows 8-15 (acc 3 odd, acc 2 even chunks from lane l ^ 8)
      const bool lo = (threadIdx.x & 15) < 8;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float s1 = __shfl_xor(acc[1][i], 8), s2 = __shfl_xor(acc[2][i], 8);
        o[i] = lo ? acc[0][i] + s1 : acc[3][i] + s2;
      }
    }
#pragma unroll
    for (int k = 0; k < NA; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};
    return o;
  }

  // 32-column tile (four row groups): columns 16 SUB .. 16 SUB + 15 from
  // accumulators 4 SUB .. 4 SUB + 3, combined as fold does for two groups;
  // the accumulators are left as they are
  template <int SUB>
  __device__ __forceinline__ static f32x4 fold_sub(const f32x4 (&acc)[NA]) {
    static_assert(NR == 4 && SUB < 2, "32-column tiles");
    const bool lo = (threadIdx.x & 15) < 8;
    f32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float s1 = __shfl_xor(acc[4 * SUB + 1][i], 8), s2 = __shfl_xor(acc[4 * SUB + 2][i], 8);
      o[i] = lo ? acc[4 * SUB][i] + s1 : acc[4 * SUB + 3][i] + s2;
    }
    return o;
  }
};

// Tile finished: sum the 16 waves' partial tiles in wave order, run the epilogue.
template <typename T, int EPI, int TW>
__device__ __forceinline__ void s_finish_tile(const GemmArgs &a, f32x4 &acc, float (*red)[256], float *ct, int t,
                                              int layer, float *best_v, int *best_i, const double *inv_freq,
                                              const EpiPre &pre, bool first) {
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
  s_epilogue<T, EPI, TW>(a, ct, t, layer, best_v, best_i, inv_freq, pre, first);
}

// Split pair (residual projection, 32-column tile, one half of K per
// workgroup): the waves' partials of the tile's two 16-column halves are summed
// in wave order into cts[0..511]; the sum goes to this half's slice of
// a.spart, and the second workgroup of the pair to arrive (counter a.cnt[cg])
// adds half 0 + half 1, in that order whichever half arrives second, to the
// residual and clears the counter for the next launch.  The first to arrive
// only leaves its partial: no workgroup waits for another.  Every value that
// crosses workgroups (partials, counter) moves through device-scope atomic
// accesses, each coherent across the XCDs by itself; every wave waits until
// its partial stores have completed before the barrier that precedes the
// counter increment, and the second workgroup issues its loads after its
// increment has returned.  Device-scope release/acquire fences instead write
// back and invalidate the XCD's whole L2: the projection took 29.7 us with
// one such pair per workgroup and 73.5 us with one per wave, against 25.4 us
// (Qwen3-8B shape, K 12288, measured).
// s_waitcnt vmcnt(0) (gfx9 encoding: expcnt and lgkmcnt at their maxima, so
// only vector-memory operations are waited for)
constexpr int kWaitVmem = 0x0F70;

template <typename T>
__device__ __forceinline__ void s_finish_split(const GemmArgs &a, const f32x4 (&acc2)[2], float (*red)[256],
                                               float *cts, int cg, int half, float xpre, int *s_old) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
#pragma unroll
  for (int sub = 0; sub < 2; ++sub) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(4 * g + i) * 16 + ln] = f4get(acc2[sub], i);
    lds_barrier();
    if (tid < 256) {
      float sm = 0.f;
#pragma unroll
      for (int w = 0; w < kSWaves; ++w) sm += red[w][tid];
      cts[256 * sub + tid] = sm;
    }
    lds_barrier();
  }
  const int r = (tid >> 4) & 15, col = cg * 32 + 16 * ((tid >> 8) & 1) + (tid & 15);
  const bool mine = tid < 512 && r < a.M;
  const float v = tid < 512 ? cts[tid] : 0.f;
  if (mine) __hip_atomic_store(a.spart + ((size_t)half * 16 + r) * a.N + col, v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(kWaitVmem);   // this wave's partial stores have completed
  __syncthreads();
  if (tid == 0) *s_old = (int)__hip_atomic_fetch_add(a.cnt + cg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (*s_old == 1) {   // second to arrive (uniform)
    if (mine) {
      const float o = __hip_atomic_load(a.spart + ((size_t)(1 - half) * 16 + r) * a.N + col, __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT);
      const float p0 = half == 0 ? v : o, p1 = half == 0 ? o : v;
      a.X[(size_t)r * a.ldx + col] = xpre + (p0 + p1);
    }
    if (tid == 0) __hip_atomic_store(a.cnt + cg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// A_COPY_ROWS (residual projection and LM head argmax): grid.y is a 16-row
// group; the activation and residual rows move to the group's first row and M
// becomes the group's row count (at most 16).  Field by field, so the
// arguments stay in registers.
template <typename T>
__device__ __forceinline__ GemmArgs row_slice(const GemmArgs &a0) {
  GemmArgs a = a0;
  const int r0 = 16 * (int)blockIdx.y;
  a.row0 = r0;
  a.M = min(16, a0.M - r0);
  a.A = (const T *)a0.A + (size_t)r0 * a0.lda;
  if (a0.X) a.X = a0.X + (size_t)r0 * a0.ldx;
  return a;
}

// FLAT: the weight slices of a.z_flat layers form one tile range (the
// inject's per-layer K/V projections); otherwise grid.y selects the slice.
template <typename T, int EPI, int AM, int TW = 16, bool FLAT = false>
__global__ __launch_bounds__(kSThreads) void gemm_stream_kernel(const GemmArgs a0) {
  static_assert(AM != A_COPY_ROWS || EPI == EPI_RESID || EPI == EPI_ARGMAX,
                "row groups serve the residual projection and the LM head");
  // TW = 32: the split pair of the residual projection (one workgroup per
  // pair half, grid = 2 x the 32-column tiles, a multiple of 16)
  constexpr bool SPLIT = TW == 32;
  static_assert(!SPLIT || (EPI == EPI_RESID && AM == A_GLOBAL && !FLAT), "split pairs: residual projection");
  // grid.y is the weight slice (layer), or the 16-row group of A_COPY_ROWS
  constexpr bool ROWS = AM == A_COPY_ROWS;
  const int layer = ROWS ? 0 : blockIdx.y;
  const GemmArgs a = ROWS ? row_slice<T>(a0) : a0;
  constexpr bool RES = AM != A_GLOBAL;
  constexpr int KR = stream_res_k<T>();                        // resident k capacity
  constexpr int ASTR = (RES ? KR : 0) * (int)sizeof(T) + 16;   // bytes per resident row
  // 1 KB loads per batch (the double-buffered fragments stay within 64 VGPRs)
  constexpr int U = TW == 8 ? 4 : (RES ? 8 : 4) / (int)(sizeof(T) / 2);
  using Buf = StreamBuf<T, U, RES, TW>;
  __shared__ __align__(16) unsigned char a_lds[RES ? 16 * ASTR : 16];
  __shared__ float red[kSWaves][256];
  __shared__ float ct[SPLIT ? 512 : 256];
  __shared__ int s_old;
  __shared__ double inv_freq[64];   // RoPE inverse frequencies (head_dim <= 128)
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, ln = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  EpiPre pre{0.f, 0, 0};   // set below, before the staging loads
  // RoPE inverse frequencies, computed once the first loads are in flight;
  // the barriers of the staging and of every tile's reduction publish them
  // before the first epilogue reads them.  With a cache copy (target verify)
  // the page of the thread's row position is read here too, behind the
  // staging and weight loads, so no wait holds them back.
  auto init_rope = [&]() {
    if constexpr (qkv_epi(EPI) || EPI == EPI_INJECT) {
      if (tid < a.hd / 2) inv_freq[tid] = rope_inv_freq(tid, a.hd, a.log2_theta);
    }
    if constexpr (EPI == EPI_QKV_CACHE) {
      {
        const int r = min(tid / (TW / 2), a.M - 1);
        pre.page = a.block_table[(size_t)(r / a.block_size) * a.max_pages +
                                 (pre.ctx + r % a.block_size) / a.page_size];
      }
    }
  };
  // FLAT: tile t is tile t % n_groups of slice t / n_groups, so a workgroup
  // stages its rows once for tiles of several slices
  // SPLIT: workgroup u takes half (u / 8) % 2 of K for 32-column tile
  // (u % 8) + 8 (u / 16), so the two halves of a tile run on one XCD
  // (workgroups u and u + 8) and share its L2
  const int KH = SPLIT ? a.K / 2 : a.K;                        // K of one workgroup's range
  const int half = SPLIT ? ((int)blockIdx.x >> 3) & 1 : 0;
  const T *W0 = (const T *)a0.W[layer];
  auto slice_of = [&](int t) { return FLAT ? t / a.n_groups : layer; };
  auto tile_in = [&](int t) {
    return FLAT ? t - (t / a.n_groups) * a.n_groups : SPLIT ? (t & 7) | ((t >> 4) << 3) : t;
  };
  auto w_of = [&](int t) {
    return FLAT ? (const T *)a0.W[slice_of(t)] : SPLIT ? W0 + (size_t)((t >> 3) & 1) * KH : W0;
  };
  const int ntiles = FLAT ? a.n_groups * a.z_flat : a.n_groups;
  const int CPT = KH / Buf::CE;                                // chunk steps per tile
  const int CPW = (CPT + kSWaves - 1) / kSWaves;               // chunks per wave
  const int cbeg = min(CPT, wave * CPW), cend = min(CPT, cbeg + CPW);
  const int clast = CPT - 1;                                   // always a valid chunk
  const int nb = (CPW + Buf::S - 1) / Buf::S;                  // batches per tile per wave
  const int my_tiles = blockIdx.x < ntiles ? (ntiles - 1 - blockIdx.x) / gridDim.x + 1 : 0;
  const int total = my_tiles * nb;
  // tile of batch q of this workgroup, clamped to a valid tile
  const int grid = gridDim.x;
  auto tile_of = [&](int q) { return min((int)blockIdx.x + (q / nb) * grid, ntiles - 1); };

  // batch Q: its tile and first chunk, or the dummy read past the end
#define DF_ISSUE(BUF, Q)                                                                        \
  {                                                                                            \
    const bool live_ = (Q) < total;                                                            \
    const int d_ = min(cbeg, clast); /* the dummy's chunk, valid even for a wave with no chunks */ \
    const int t_ = tile_of(live_ ? (Q) : 0);                                                      \
    BUF.template issue<EPI>(a, w_of(t_), arow, arow_hi, tile_in(t_), live_ ? cbeg + ((Q) % nb) * Buf::S : d_, \
                            live_ ? clast : d_);                                               \
  }
  pre = s_epi_pre<EPI, TW>(a, tile_in(tile_of(0)));
  const T *A = (const T *)a.A;
  // activation pointer of this lane: rows in LDS, or rows in global memory
  // (bf16: whole lines, rows ln % 8 and 8 + ln % 8 at chunk 2c + ln / 8; rows
  // >= M read row 0 and are never stored)
  const T *arow, *arow_hi = nullptr;
  if constexpr (RES) {
    arow = reinterpret_cast<const T *>(a_lds + ln * ASTR) + 8 * g;
  } else if constexpr (Buf::WL) {
    const int r0 = ln & 7, r1 = 8 + (ln & 7);
    arow = A + (size_t)(r0 < a.M ? r0 : 0) * a.lda + (size_t)half * KH + 8 * g + 32 * (ln >> 3);
    arow_hi = A + (size_t)(r1 < a.M ? r1 : 0) * a.lda + (size_t)half * KH + 8 * g + 32 * (ln >> 3);
  } else {
    arow = A + (size_t)(ln < a.M ? ln : 0) * a.lda + 8 * g;
  }
  Buf bufa, bufb;

  // ---- resident activation rows ---------------------------------------------
  // Wave w stages row w.  Every load of the row (and of the gain) is issued
  // unconditionally, from clamped addresses.  The first weight batch follows
  // once the wave's row has landed: issued together, the batch's HBM requests
  // held the row's L2 hits back (rows landed ~7.5 us after launch instead of
  // ~2.9 us, measured; the step got 18 us faster).  Rows >= M are stored as
  // zeros.
  if constexpr (RES) {
    const int r = wave;
    const bool have_row = r < a.M;
    const int rr = min(r, a.M - 1);
    if constexpr (AM == A_COPY || AM == A_COPY_ROWS) {
      // the row goes through registers (NV 16-byte pieces per lane, all
      // issued first, clamped source); the first weight batch is issued once
      // the row is written to LDS
      constexpr int EPV = 16 / (int)sizeof(T);     // elements per 16-byte vector
      constexpr int NV = KR / EPV / 64;            // vectors per lane at most
      const int nvec = a.K / EPV;
      const uint4 *src = reinterpret_cast<const uint4 *>(A + (size_t)rr * a.lda);
      uint4 cv[NV];
#pragma unroll
      for (int k = 0; k < NV; ++k) cv[k] = src[min(lane + 64 * k, nvec - 1)];
      init_rope();
      // every piece of the LDS row is written (zeros past K and for rows >= M):
      // no branch per piece keeps this once-per-launch code short
      uint4 *dst = reinterpret_cast<uint4 *>(a_lds + r * ASTR);
#pragma unroll
      for (int k = 0; k < NV; ++k) {
        const int i = lane + 64 * k;
        dst[i] = have_row && i < nvec ? cv[k] : make_uint4(0, 0, 0, 0);
      }
      DF_ISSUE(bufa, 0);
      lds_barrier();
    } else {
      // lane owns the 4-element groups q4 = lane + 64 k of the row; the gain
      // is read once per workgroup (one group per thread, issued first) and
      // parked in the reduction buffer, which is unused until the first tile
      // finishes.  The gain is published before the rows land, so each wave
      // normalises its row as soon as that row arrives (rows reach a compute
      // unit one group of four waves after another, not all at once).
      constexpr int PQ = KR / 4 / 64;              // groups per lane at most
      const int nq4 = a.K / 4;
      const float4 gq = load4((const T *)a.gain, min(tid, nq4 - 1));
      float4 xv[PQ];
      if constexpr (AM == A_EMBED_NORM) {
        const int s = rr / a.block_size, j = rr - s * a.block_size;
        const int id = a.ids ? a.ids[rr] : (j == 0 ? a.anchor[s] : a.mask_id);
        const T *erow = (const T *)a.embed + (size_t)id * a.K;
#pragma unroll
        for (int k = 0; k < PQ; ++k) xv[k] = load4(erow, min(lane + 64 * k, nq4 - 1));
      } else {
        const float4 *x4 = reinterpret_cast<const float4 *>(a.X + (size_t)rr * a.ldx);
#pragma unroll
        for (int k = 0; k < PQ; ++k) xv[k] = x4[min(lane + 64 * k, nq4 - 1)];
      }
      init_rope();
      // groups past K hold zeros (row values and gain alike), so the loops
      // below run branch-free over the whole LDS row: this once-per-launch
      // code stays short
      float4 *gl = reinterpret_cast<float4 *>(&red[0][0]);
      if (tid < KR / 4) gl[tid] = tid < nq4 ? gq : make_float4(0.f, 0.f, 0.f, 0.f);
      lds_barrier();                               // gain visible
      float ss = 0.f;
#pragma unroll
      for (int k = 0; k < PQ; ++k) {
        if (lane + 64 * k >= nq4) xv[k] = make_float4(0.f, 0.f, 0.f, 0.f);
        ss += xv[k].x * xv[k].x;
        ss += xv[k].y * xv[k].y;
        ss += xv[k].z * xv[k].z;
        ss += xv[k].w * xv[k].w;
      }
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) ss += __shfl_xor(ss, o);
      DF_ISSUE(bufa, 0);   // the row has landed
      const float rs = 1.0f / sqrtf(ss / (float)a.K + a.eps);
      const float rsr = have_row ? rs : 0.f;       // rows >= M are stored as zeros
      T *dst = reinterpret_cast<T *>(a_lds + r * ASTR);
#pragma unroll
      for (int k = 0; k < PQ; ++k) {
        const int q4 = lane + 64 * k;
        const float4 gv = gl[q4];
        float4 o;
        o.x = xv[k].x * rsr * gv.x;
        o.y = xv[k].y * rsr * gv.y;
        o.z = xv[k].z * rsr * gv.z;
        o.w = xv[k].w * rsr * gv.w;
        store4(dst, q4, o);
      }
      if (AM == A_EMBED_NORM && have_row && blockIdx.x == 0 && layer == 0) {
        // one workgroup starts the residual stream with the embedding rows
#pragma unroll
        for (int k = 0; k < PQ; ++k) {
          const int q4 = lane + 64 * k;
          if (q4 < nq4) reinterpret_cast<float4 *>(a.X + (size_t)r * a.ldx)[q4] = xv[k];
        }
      }
      lds_barrier();
    }
  } else {
    DF_ISSUE(bufa, 0);
    init_rope();
  }

  float best_v = -INFINITY;
  int best_i = -1;   // set by the first tile
  f32x4 accs[Buf::NA];
#pragma unroll
  for (int k = 0; k < Buf::NA; ++k) accs[k] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 acc;
  auto finish = [&](int qq, bool first) {
    const int tf = tile_of(qq);
    if constexpr (SPLIT) {
      const f32x4 a2[2] = {Buf::template fold_sub<0>(accs), Buf::template fold_sub<1>(accs)};
      s_finish_split<T>(a, a2, red, ct, tile_in(tf), half, pre.x, &s_old);
    } else {
      acc = Buf::fold(accs);
      s_finish_tile<T, EPI, TW>(a, acc, red, ct, tile_in(tf), slice_of(tf), &best_v, &best_i, inv_freq, pre, first);
    }
  };
  // static ping-pong between two register buffers (dynamic selection would
  // spill the fragments to scratch): the next batch is issued before the
  // current one is consumed.  Every batch is issued whether or not it exists
  // (past the end it re-reads the wave's first chunk of the workgroup's first
  // tile, a cache hit, and is never used): with no branch around the issue,
  // consuming one buffer waits for that buffer only.  Both halves always run
  // (no exit in the middle of the loop keeps the count of outstanding loads
  // identical on every path into the loop head); a second half past the end
  // consumes a dummy batch and finishes nothing.
  for (int q = 0; q < total; q += 2) {
    DF_ISSUE(bufb, q + 1);
    bufa.compute(accs, arow, cbeg + (q % nb) * Buf::S, cend, clast);
    if (q % nb == nb - 1) finish(q, q < nb);
    DF_ISSUE(bufa, q + 2);
    bufb.compute(accs, arow, cbeg + ((q + 1) % nb) * Buf::S, cend, clast);
    if ((q + 1) % nb == nb - 1 && q + 1 < total) finish(q + 1, q + 1 < nb);
  }
#undef DF_ISSUE

  if constexpr (EPI == EPI_ARGMAX) {
    if (tid < 16 && tid < a.M) {
      a.amax_val[(size_t)(a.row0 + tid) * gridDim.x + blockIdx.x] = best_v;
      a.amax_idx[(size_t)(a.row0 + tid) * gridDim.x + blockIdx.x] = best_i;
    }
  }
}

// K longer than the resident capacity: one 16-column tile per workgroup, the
// activation rows staged into LDS one K-portion at a time.  A portion has
// KR / 32 k-chunks, exactly one batch of U chunks per wave.  While portion p
// is multiplied, the rows of portion p + 1 (registers) and its weight batch
// are already in flight; the accumulator stays in registers until the whole K
// is done.
template <typename T, int EPI>
__global__ __launch_bounds__(kSThreads) void gemm_portion_kernel(const GemmArgs a) {
  const int layer = blockIdx.y;
  constexpr int KR = stream_res_k<T>();
  constexpr int ASTR = KR * (int)sizeof(T) + 16;
  constexpr int U = 8 / (int)(sizeof(T) / 2);
  constexpr int EPV = 16 / (int)sizeof(T);       // elements per 16-byte vector
  constexpr int CPP = KR / 32;                   // chunks per full portion
  constexpr int NV = KR / EPV / 64;              // staged vectors per lane
  static_assert(CPP == kSWaves * U, "one batch per wave per portion");
  __shared__ __align__(16) unsigned char a_lds[16 * ASTR];
  __shared__ float red[kSWaves][256];
  __shared__ float ct[256];
  __shared__ double inv_freq[64];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, ln = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int t = blockIdx.x;
  if constexpr (qkv_epi(EPI) || EPI == EPI_INJECT) {
    if (tid < a.hd / 2) inv_freq[tid] = rope_inv_freq(tid, a.hd, a.log2_theta);
  }
  const T *W = (const T *)a.W[layer];
  const int nchunk = a.K / 32;
  const int np = (nchunk + CPP - 1) / CPP;       // portions
  const int clast = nchunk - 1;
  const T *wrow = W + (size_t)s_weight_row<EPI, 16>(a, t, ln) * a.ldw + 8 * g;
  const T *arow = reinterpret_cast<const T *>(a_lds + ln * ASTR) + 8 * g;
  // wave w stages row w (row 0 stands in for rows >= M, stored as zeros)
  const bool have_row = wave < a.M;
  const uint4 *srow = reinterpret_cast<const uint4 *>((const T *)a.A + (size_t)min(wave, a.M - 1) * a.lda);
  uint4 *drow = reinterpret_cast<uint4 *>(a_lds + wave * ASTR);
  // portion p: its first chunk and chunk count; past the last portion a dummy
  // re-read of the tile's chunk 0 (a cache hit, never used) keeps the issue
  // free of branches
  auto pfirst = [&](int p) { return p < np ? p * CPP : 0; };
  auto pcount = [&](int p) { return p < np ? min(CPP, nchunk - p * CPP) : 1; };
  const EpiPre pre = s_epi_pre<EPI, 16>(a, t);

  Frag<T> wa[U], wb[U];
  uint4 cv[NV];
#define DF_PORTION_LOAD(WBUF, P)                                                              \
  {                                                                                          \
    const int f_ = pfirst(P), n_ = pcount(P) * 32 / EPV;                                     \
    _Pragma("unroll") for (int k = 0; k < NV; ++k) cv[k] = srow[f_ * 32 / EPV + min(lane + 64 * k, n_ - 1)]; \
    const int c0_ = (P) < np ? f_ + wave * U : 0, cl_ = (P) < np ? clast : 0;                 \
    _Pragma("unroll") for (int j = 0; j < U; ++j) WBUF[j].load(wrow + 32 * min(c0_ + j, cl_)); \
    __builtin_amdgcn_sched_barrier(0);  /* keep the prefetch ahead of the products */       \
  }
#define DF_PORTION_STORE(P)                                                                   \
  {                                                                                          \
    const int n_ = pcount(P) * 32 / EPV;                                                     \
    _Pragma("unroll") for (int k = 0; k < NV; ++k) {                                         \
      const int i_ = lane + 64 * k;                                                          \
      if (i_ < n_) drow[i_] = have_row ? cv[k] : make_uint4(0, 0, 0, 0);                     \
    }                                                                                        \
  }
#define DF_PORTION_MMA(WBUF, P)                                                               \
  {                                                                                          \
    const int pc_ = pcount(P), b_ = min(pc_, wave * U), e_ = min(pc_, b_ + U);               \
    _Pragma("unroll") for (int j = 0; j < U; ++j) {                                          \
      Frag<T> wj = WBUF[j], af;                                                              \
      if (b_ + j >= e_) wj.zero();                                                           \
      af.load(arow + 32 * min(b_ + j, pc_ - 1));                                             \
      acc = mma(acc, af, wj);                                                                \
    }                                                                                        \
  }

  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  DF_PORTION_LOAD(wa, 0);
  DF_PORTION_STORE(0);
  lds_barrier();
  for (int p = 0; p < np; p += 2) {
    DF_PORTION_LOAD(wb, p + 1);
    DF_PORTION_MMA(wa, p);
    if (p + 1 >= np) break;
    lds_barrier();
    DF_PORTION_STORE(p + 1);
    lds_barrier();
    DF_PORTION_LOAD(wa, p + 2);
    DF_PORTION_MMA(wb, p + 1);
    if (p + 2 >= np) break;
    lds_barrier();
    DF_PORTION_STORE(p + 2);
    lds_barrier();
  }
#undef DF_PORTION_LOAD
#undef DF_PORTION_STORE
#undef DF_PORTION_MMA
  float best_v = -INFINITY;
  int best_i = -1;   // set by the first tile
  s_finish_tile<T, EPI, 16>(a, acc, red, ct, t, layer, &best_v, &best_i, inv_freq, pre, true);
  if constexpr (EPI == EPI_ARGMAX) {
    if (tid < 16 && tid < a.M) {
      a.amax_val[(size_t)(a.row0 + tid) * gridDim.x + blockIdx.x] = best_v;
      a.amax_idx[(size_t)(a.row0 + tid) * gridDim.x + blockIdx.x] = best_i;
    }
  }
}

template <typename T, int EPI>
static hipError_t launch_s(int am, const GemmArgs &a, dim3 grid, hipStream_t st) {
  const dim3 block(kSThreads);
  if (a.z_flat > 0) {   // one flat tile range over the layers: the inject's K/V projections
    if constexpr (EPI == EPI_INJECT) {
      switch (am) {
        case A_COPY: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_COPY, 16, true>), grid, block, 0, st, a); break;
        case A_GLOBAL:
          hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_GLOBAL, 16, true>), grid, block, 0, st, a);
          break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (am == A_SPLIT2) {   // split pairs: bf16 residual projection, activations from global memory
    if constexpr (sizeof(T) == 2 && EPI == EPI_RESID) {
      hipLaunchKernelGGL((gemm_stream_kernel<T, EPI_RESID, A_GLOBAL, 32>), grid, block, 0, st, a);
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  if (am & A_TW8) {   // 8-column tiles: bf16 QKV with RMSNorm staging only
    if constexpr (sizeof(T) == 2 && qkv_epi(EPI)) {
      switch (am & ~A_TW8) {
        case A_NORM: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_NORM, 8>), grid, block, 0, st, a); break;
        case A_EMBED_NORM:
          hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_EMBED_NORM, 8>), grid, block, 0, st, a);
          break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    } else {
      return hipErrorInvalidValue;
    }
  }
  switch (am) {
    case A_GLOBAL: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_GLOBAL>), grid, block, 0, st, a); break;
    case A_COPY: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_COPY>), grid, block, 0, st, a); break;
    case A_NORM: hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_NORM>), grid, block, 0, st, a); break;
    case A_EMBED_NORM:
      hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_EMBED_NORM>), grid, block, 0, st, a);
      break;
    case A_COPY_ROWS:   // grid.y = 16-row groups
      if constexpr (EPI == EPI_RESID || EPI == EPI_ARGMAX) {
        hipLaunchKernelGGL((gemm_stream_kernel<T, EPI, A_COPY_ROWS>), grid, block, 0, st, a);
        break;
      } else {
        return hipErrorInvalidValue;
      }
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
    case EPI_QKV_CACHE: return launch_s<T, EPI_QKV_CACHE>(am, a, grid, st);
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
