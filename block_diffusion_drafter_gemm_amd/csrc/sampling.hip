// Verification at temperature > 0 (the speculative-sampling rule of standard
// speculative decoding, [FN] §1): Gumbel-max draws from softmax(z / T) with the
// log-sum-exp of every row, and the accept / resample step over the drafter's
// and the target's logits.
//
// Random numbers: Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel
// random numbers: as easy as 1, 2, 3", SC 2011), keyed by the caller's 64-bit
// seed; the counter is (column / 4, row, offset, tag) and the draw for column c
// is word c mod 4, turned into u = (floor(w / 2^9) + 1/2) * 2^-23 in (0, 1).
// One Philox call serves four consecutive columns of one thread.
//
// Vocabulary passes are split into 1024-column chunks (4 columns, one 16-byte
// load and one Philox call per thread of a 256-thread workgroup); a workgroup
// takes 1 to 8 consecutive chunks of one row so that many rows do not launch
// tens of thousands of tiny workgroups.  A per-row merge follows; the logits
// are read once per pass (fp32, [rows, V] row-major).
#include <algorithm>
#include <climits>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

namespace {

constexpr uint32_t kTagAccept = 0xFFFFFFFEu;     // acceptance uniforms
constexpr uint32_t kTagResidual = 0xFFFFFFFFu;   // residual draws

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    // one 32 x 32 -> 64-bit product each (high and low words)
    const uint64_t p0 = (uint64_t)0xD2511F53u * c.x, p1 = (uint64_t)0xCD9E8D57u * c.z;
    c = make_uint4((uint32_t)(p1 >> 32) ^ c.y ^ k0, (uint32_t)p1, (uint32_t)(p0 >> 32) ^ c.w ^ k1, (uint32_t)p0);
  }
  return c;
}

__device__ __forceinline__ float word_of(const uint4 &w, int j) {
  const uint32_t x = j == 0 ? w.x : j == 1 ? w.y : j == 2 ? w.z : w.w;
  return ((float)(x >> 9) + 0.5f) * 0x1p-23f;    // exact in fp32, in (0, 1)
}

// Keys and log-sum-exp terms are kept in base 2 (the hardware's log2 / exp2;
// a few ulp, against near-ties at 1e-4): with y = z * log2(e) / T, the
// Gumbel-max key (z/T + g) * log2(e) is y - log2(-log2 u) up to a constant
// shared by all columns, and lse = ln 2 * (max y + log2 sum 2^(y - max y)).
constexpr float kLog2e = 1.4426950408889634f, kLn2 = 0.6931471805599453f;
__device__ __forceinline__ float log2_hw(float x) { return __builtin_amdgcn_logf(x); }
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float gumbel2(float u) { return -log2_hw(-log2_hw(u)); }

// 4 logits of one thread from column c0 (one 16-byte load when the row is
// 16-byte aligned)
__device__ __forceinline__ float4 load4_cols(const float *z, int c0, int vocab) {
  if ((vocab & 3) == 0 && (reinterpret_cast<uintptr_t>(z) & 15) == 0) return *reinterpret_cast<const float4 *>(z + c0);
  float4 v;
  v.x = z[c0];
  v.y = c0 + 1 < vocab ? z[c0 + 1] : 0.f;
  v.z = c0 + 2 < vocab ? z[c0 + 2] : 0.f;
  v.w = c0 + 3 < vocab ? z[c0 + 3] : 0.f;
  return v;
}

__device__ __forceinline__ float f4at(const float4 &v, int j) { return j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w; }

// (key, lowest index) and (max, sum of 2^(y - max)) of one thread or group
struct Part {
  float key;
  int idx;
  float m;
  float s;
};

__device__ __forceinline__ void merge(Part &a, const Part &b) {
  if (b.key > a.key || (b.key == a.key && b.idx < a.idx)) {
    a.key = b.key;
    a.idx = b.idx;
  }
  const float m = fmaxf(a.m, b.m);
  if (m != -INFINITY) {
    a.s = a.s * exp2f(a.m - m) + b.s * exp2f(b.m - m);
    a.m = m;
  }
}

__device__ __forceinline__ Part wave_merge(Part p) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    Part q;
    q.key = __shfl_xor(p.key, o);
    q.idx = __shfl_xor(p.idx, o);
    q.m = __shfl_xor(p.m, o);
    q.s = __shfl_xor(p.s, o);
    merge(p, q);
  }
  return p;
}

// Merge of a 256-thread workgroup; thread 0 holds the result.
__device__ __forceinline__ Part block_merge(Part p) {
  __shared__ Part red[4];
  p = wave_merge(p);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = p;
  __syncthreads();
  if (threadIdx.x == 0)
    for (int w = 1; w < 4; ++w) merge(p, red[w]);
  return p;
}

__device__ __forceinline__ Part empty_part() { return Part{-INFINITY, INT_MAX, -INFINITY, 0.f}; }

// Chunks g*per .. g*per + per - 1 of row r: Gumbel-max key z/T + g and the
// log-sum-exp terms.  All of a thread's loads are issued before the first
// Philox call; a thread's columns increase, so a strict comparison keeps the
// lowest id.
constexpr int kSamplePer = 8;   // most chunks per workgroup

__global__ __launch_bounds__(256) void sample_partial_kernel(const float *logits, int vocab, float scale,
                                                             uint32_t k0, uint32_t k1, uint32_t offset,
                                                             uint32_t tag, int per, Part *part) {
  const int r = blockIdx.x, g = blockIdx.y;
  const float *z = logits + (size_t)r * vocab;
  float4 zv[kSamplePer];
  float m = -INFINITY;
#pragma unroll
  for (int it = 0; it < kSamplePer; ++it) {
    const int c0 = (g * per + it) * kSampleCols + (int)threadIdx.x * 4;
    if (it < per && c0 < vocab) {
      zv[it] = load4_cols(z, c0, vocab);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (c0 + j < vocab) m = fmaxf(m, f4at(zv[it], j) * scale);
    }
  }
  Part p = empty_part();
  p.m = m;
#pragma unroll
  for (int it = 0; it < kSamplePer; ++it) {
    const int c0 = (g * per + it) * kSampleCols + (int)threadIdx.x * 4;
    if (it < per && c0 < vocab) {
      const uint4 w = philox4x32_10(make_uint4((uint32_t)c0 >> 2, (uint32_t)r, offset, tag), k0, k1);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (c0 + j < vocab) {
          const float y = f4at(zv[it], j) * scale;
          p.s += exp2_hw(y - m);
          const float key = y + gumbel2(word_of(w, j));
          const bool better = key > p.key;     // increasing column: keeps the lowest id
          p.key = better ? key : p.key;
          p.idx = better ? c0 + j : p.idx;
        }
      }
    }
  }
  p = block_merge(p);
  if (threadIdx.x == 0) part[(size_t)r * gridDim.y + g] = p;
}

// One wave per row: merge the chunk partials into the drawn id and the lse.
__global__ __launch_bounds__(64) void sample_reduce_kernel(const Part *part, int n_chunks, int *ids_out,
                                                           float *lse_out) {
  const int r = blockIdx.x;
  Part p = empty_part();
  for (int i = threadIdx.x; i < n_chunks; i += 64) merge(p, part[(size_t)r * n_chunks + i]);
  p = wave_merge(p);
  if (threadIdx.x == 0) {
    ids_out[r] = p.idx;
    if (lse_out) lse_out[r] = kLn2 * (p.m + log2f(p.s));
  }
}

struct AcceptArgs {
  const float *dz, *dlse;   // drafter logits [batch*(B-1), V], lse [batch*(B-1)]
  const int *dids;          // drafts [batch, B-1]
  const float *tz, *tlse;   // target logits [batch*B, V], lse [batch*B]
  const int *tids;          // the target's own draws [batch, B]
  const int *block_len;
  int B, vocab;
  float inv_t;
  uint32_t k0, k1, offset;
};

// Index of the first rejected draft of sequence s (0-based), or bs - 1 when
// every draft is kept.  Run by one whole wave.  Draft i is kept when
// u_i * q_i(d_i) < p_i(d_i); an id outside the vocabulary is rejected.
__device__ __forceinline__ int first_reject(const AcceptArgs &a, int s, int bs) {
  const int i = threadIdx.x & 63;
  bool rej = false;
  if (i < bs - 1) {
    const int d = a.dids[(size_t)s * (a.B - 1) + i];
    if (d < 0 || d >= a.vocab) {
      rej = true;
    } else {
      const size_t dr = (size_t)s * (a.B - 1) + i, tr = (size_t)s * a.B + i;
      const float q = expf(a.dz[dr * a.vocab + d] * a.inv_t - a.dlse[dr]);
      const float p = expf(a.tz[tr * a.vocab + d] * a.inv_t - a.tlse[tr]);
      const uint4 w = philox4x32_10(make_uint4((uint32_t)i >> 2, (uint32_t)s, a.offset, kTagAccept), a.k0, a.k1);
      rej = !(word_of(w, i & 3) * q < p);
    }
  }
  const unsigned long long m = __ballot(rej);
  return m ? __ffsll((long long)m) - 1 : bs - 1;
}

__device__ __forceinline__ int block_len_of(const AcceptArgs &a, int s) {
  return a.block_len ? min(max(a.block_len[s], 1), a.B) : a.B;
}

// Chunk `ch` of sequence s: Gumbel-max over log max(0, p_k - q_k) at the first
// rejected position k (nothing to do when every draft is kept).
__global__ __launch_bounds__(256) void accept_partial_kernel(const AcceptArgs a, Part *part) {
  __shared__ int sk;
  const int s = blockIdx.x, ch = blockIdx.y;
  const int bs = block_len_of(a, s);
  if (threadIdx.x < 64) {
    const int k = first_reject(a, s, bs);
    if (threadIdx.x == 0) sk = k;
  }
  __syncthreads();
  const int k = sk;
  if (k == bs - 1) return;                       // all kept: the reduce takes the target's draw
  const size_t dr = (size_t)s * (a.B - 1) + k, tr = (size_t)s * a.B + k;
  const float *zd = a.dz + dr * a.vocab, *zt = a.tz + tr * a.vocab;
  const float ld = a.dlse[dr], lt = a.tlse[tr];
  Part p = empty_part();
  const int c0 = ch * kSampleCols + (int)threadIdx.x * 4;
  if (c0 < a.vocab) {
    const float4 tv = load4_cols(zt, c0, a.vocab), dv = load4_cols(zd, c0, a.vocab);
    const uint4 w = philox4x32_10(make_uint4((uint32_t)c0 >> 2, (uint32_t)s, a.offset, kTagResidual), a.k0, a.k1);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (c0 + j < a.vocab) {
        // p - q, with lse in natural-log units
        const float res = exp2_hw((f4at(tv, j) * a.inv_t - lt) * kLog2e) - exp2_hw((f4at(dv, j) * a.inv_t - ld) * kLog2e);
        const float key = res > 0.f ? log2_hw(res) + gumbel2(word_of(w, j)) : -INFINITY;
        const bool better = key > p.key;
        p.key = better ? key : p.key;
        p.idx = better ? c0 + j : p.idx;
      }
    }
  }
  p = block_merge(p);
  if (threadIdx.x == 0) part[(size_t)s * gridDim.y + ch] = p;
}

// One wave per sequence: tau and the next token.  With no positive residual
// left after fp32 rounding, the target's own draw at that position is taken.
__global__ __launch_bounds__(64) void accept_reduce_kernel(const AcceptArgs a, const Part *part, int n_chunks,
                                                           int *tau, int *bonus) {
  const int s = blockIdx.x;
  const int bs = block_len_of(a, s);
  const int k = first_reject(a, s, bs);
  if (k == bs - 1) {
    if (threadIdx.x == 0) {
      tau[s] = bs;
      bonus[s] = a.tids[(size_t)s * a.B + bs - 1];
    }
    return;
  }
  Part p = empty_part();
  for (int i = threadIdx.x; i < n_chunks; i += 64) merge(p, part[(size_t)s * n_chunks + i]);
  p = wave_merge(p);
  if (threadIdx.x == 0) {
    tau[s] = k + 1;
    bonus[s] = p.idx != INT_MAX ? p.idx : a.tids[(size_t)s * a.B + k];
  }
}

}  // namespace

size_t sample_ws_bytes(int rows, int vocab) {
  return (size_t)rows * (size_t)((vocab + kSampleCols - 1) / kSampleCols) * sizeof(Part);
}

hipError_t launch_sample(const float *logits, int rows, int vocab, float inv_t, uint64_t seed, uint32_t offset,
                         uint32_t tag, int *ids_out, float *lse_out, void *ws, hipStream_t st) {
  const int nch = (vocab + kSampleCols - 1) / kSampleCols;
  // about 2048 workgroups or more: several chunks per workgroup once rows x
  // chunks exceed that (many rows), one otherwise
  const int per = std::max(1, std::min(kSamplePer, (int)((long)rows * nch / 2048)));
  const int groups = (nch + per - 1) / per;
  Part *part = static_cast<Part *>(ws);
  hipLaunchKernelGGL(sample_partial_kernel, dim3(rows, groups), dim3(256), 0, st, logits, vocab, inv_t * kLog2e,
                     (uint32_t)seed, (uint32_t)(seed >> 32), offset, tag, per, part);
  hipLaunchKernelGGL(sample_reduce_kernel, dim3(rows), dim3(64), 0, st, part, groups, ids_out, lse_out);
  return hipGetLastError();
}

hipError_t launch_accept_sample(const float *dz, const float *dlse, const int *dids, const float *tz,
                                const float *tlse, const int *tids, int batch, int B, const int *block_len,
                                int vocab, float inv_t, uint64_t seed, uint32_t offset, int *tau, int *bonus,
                                void *ws, hipStream_t st) {
  AcceptArgs a;
  a.dz = dz;
  a.dlse = dlse;
  a.dids = dids;
  a.tz = tz;
  a.tlse = tlse;
  a.tids = tids;
  a.block_len = block_len;
  a.B = B;
  a.vocab = vocab;
  a.inv_t = inv_t;
  a.k0 = (uint32_t)seed;
  a.k1 = (uint32_t)(seed >> 32);
  a.offset = offset;
  const int nch = (vocab + kSampleCols - 1) / kSampleCols;
  Part *part = static_cast<Part *>(ws);
  hipLaunchKernelGGL(accept_partial_kernel, dim3(batch, nch), dim3(256), 0, st, a, part);
  hipLaunchKernelGGL(accept_reduce_kernel, dim3(batch), dim3(64), 0, st, a, part, nch, tau, bonus);
  return hipGetLastError();
}

}  // namespace dflash
