// Row-wise kernels of the draft step: block embedding, RMSNorm, the second
// level of the vocabulary argmax, greedy accept length and a zero fill.
#include <algorithm>

#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kNormThreads = 512;

// X[s*B + j, :] = E[j == 0 ? anchor[s] : mask] as fp32 (the residual stream).
template <typename T>
__global__ __launch_bounds__(256) void embed_kernel(const T *E, const int *anchor, int mask_id, const int *ids,
                                                    int B, int H, float *X) {
  const int row = blockIdx.x;
  const int s = row / B, j = row % B;
  const int id = ids ? ids[row] : (j == 0 ? anchor[s] : mask_id);
  const T *e = E + (size_t)id * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) X[(size_t)row * H + i] = Storage<T>::load(e, i);
}

__device__ __forceinline__ float block_sum(float v, float *red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  __syncthreads();
  if (lane == 0) red[wave] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += red[w];
  return t;
}

// Y[r] = X[src(r)] / sqrt(mean(X^2) + eps) * gain, rounded to the storage type.
// skip_anchor: output row r reads input row s*B + 1 + (r % (B-1)) with
// s = r / (B-1) (the mask rows of every block).
// One workgroup per row; each thread holds up to KV four-element groups of the
// row in registers (all loads issued at once, one pass over the row).
template <typename T, int KV>
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const float *X, const T *gain, float eps, int H, int B,
                                                               int skip_anchor, T *Y) {
  __shared__ float red[kNormThreads / 64];
  const int r = blockIdx.x, tid = threadIdx.x;
  const int src = skip_anchor ? (r / (B - 1)) * B + 1 + r % (B - 1) : r;
  const float4 *x4 = reinterpret_cast<const float4 *>(X + (size_t)src * H);
  const int n4 = H / 4;
  float4 v[KV];
#pragma unroll
  for (int k = 0; k < KV; ++k) v[k] = x4[min(tid + kNormThreads * k, n4 - 1)];
  float ss = 0.f;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    if (tid + kNormThreads * k < n4) {
      ss += v[k].x * v[k].x;
      ss += v[k].y * v[k].y;
      ss += v[k].z * v[k].z;
      ss += v[k].w * v[k].w;
    }
  }
  ss = block_sum(ss, red);
  const float rs = 1.0f / sqrtf(ss / (float)H + eps);
  T *y = Y + (size_t)r * H;
#pragma unroll
  for (int k = 0; k < KV; ++k) {
    const int q = tid + kNormThreads * k;
    if (q < n4) {
      const float4 g = load4(gain, q);
      store4(y, q, make_float4(v[k].x * rs * g.x, v[k].y * rs * g.y, v[k].z * rs * g.z, v[k].w * rs * g.w));
    }
  }
}

// Second level of the vocabulary argmax: one workgroup per row scans the
// per-column-group maxima; the lowest id wins ties.  NaN partials count as
// -inf and negative ids (a partial with no column) are skipped; the GEMM
// epilogues start every partial at a valid column, so a row with no number
// above -inf gets the lowest partial id, 0.
__global__ __launch_bounds__(256) void argmax_reduce_kernel(const float *val, const int *idx, int n_groups,
                                                            int *ids_out, float *max_out) {
  __shared__ float sv[4];
  __shared__ int si[4];
  const int r = blockIdx.x;
  float best = -INFINITY;
  int bidx = 0x7fffffff;
  for (int i = threadIdx.x; i < n_groups; i += blockDim.x) {
    const float v0 = val[(size_t)r * n_groups + i];
    const float v = v0 != v0 ? -INFINITY : v0;
    const int id = idx[(size_t)r * n_groups + i];
    if (id >= 0 && (v > best || (v == best && id < bidx))) { best = v; bidx = id; }
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(best, o);
    const int oi = __shfl_xor(bidx, o);
    if (ov > best || (ov == best && oi < bidx)) { best = ov; bidx = oi; }
  }
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  if (lane == 0) { sv[wave] = best; si[wave] = bidx; }
  __syncthreads();
  if (threadIdx.x == 0) {
    for (int w = 1; w < (int)(blockDim.x >> 6); ++w)
      if (sv[w] > best || (sv[w] == best && si[w] < bidx)) { best = sv[w]; bidx = si[w]; }
    ids_out[r] = bidx == 0x7fffffff ? 0 : bidx;   // n_groups >= 1: always set
    if (max_out) max_out[r] = best;
  }
}

// One wave per sequence: tau = 1 + (leading matches of draft vs target), bonus = target[tau-1].
__global__ __launch_bounds__(64) void accept_kernel(const int *draft, const int *target, int B,
                                                    const int *block_len, int *tau, int *bonus) {
  const int s = blockIdx.x, lane = threadIdx.x;
  const int bs = block_len ? min(max(block_len[s], 1), B) : B;   // this sequence's block size
  const bool miss = lane < bs - 1 && draft[(size_t)s * (B - 1) + lane] != target[(size_t)s * B + lane];
  const unsigned long long m = __ballot(miss);
  const int k = m ? __ffsll((long long)m) - 1 : bs - 1;
  if (lane == 0) {
    tau[s] = k + 1;
    bonus[s] = target[(size_t)s * B + k];
  }
}

__global__ void zero_kernel(uint4 *p, size_t n16) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

hipError_t launch_embed(bool is_bf16, const void *embed, const int *anchor, int mask_id, const int *ids, int batch,
                        int B, int H, float *X, hipStream_t st) {
  if (is_bf16)
    hipLaunchKernelGGL(embed_kernel<bf16_t>, dim3(batch * B), dim3(256), 0, st, (const bf16_t *)embed, anchor,
                       mask_id, ids, B, H, X);
  else
    hipLaunchKernelGGL(embed_kernel<float>, dim3(batch * B), dim3(256), 0, st, (const float *)embed, anchor,
                       mask_id, ids, B, H, X);
  return hipGetLastError();
}

// One workgroup per block row: its K and V rows (kvd elements each) go to the
// paged slot of position ctx_len[s] + j (page from the sequence's table).
template <typename T>
__global__ __launch_bounds__(256) void kv_append_kernel(const T *kb, const T *vb, T *kc, T *vc, const int *block_table,
                                                        const int *ctx_len, int B, int kvd, int max_pages,
                                                        int page_size) {
  const int row = blockIdx.x, s = row / B, j = row % B;
  const int pos = ctx_len[s] + j;
  const int page = block_table[(size_t)s * max_pages + pos / page_size];
  const size_t dst = ((size_t)page * page_size + pos % page_size) * kvd;
  for (int i = threadIdx.x; i < kvd; i += blockDim.x) {
    kc[dst + i] = kb[(size_t)row * kvd + i];
    vc[dst + i] = vb[(size_t)row * kvd + i];
  }
}

hipError_t launch_kv_append(bool is_bf16, const void *kb, const void *vb, void *kc, void *vc, const int *block_table,
                            const int *ctx_len, int batch, int B, int kvd, int max_pages, int page_size,
                            hipStream_t st) {
  if (is_bf16)
    hipLaunchKernelGGL(kv_append_kernel<bf16_t>, dim3(batch * B), dim3(256), 0, st, (const bf16_t *)kb,
                       (const bf16_t *)vb, (bf16_t *)kc, (bf16_t *)vc, block_table, ctx_len, B, kvd, max_pages,
                       page_size);
  else
    hipLaunchKernelGGL(kv_append_kernel<float>, dim3(batch * B), dim3(256), 0, st, (const float *)kb,
                       (const float *)vb, (float *)kc, (float *)vc, block_table, ctx_len, B, kvd, max_pages,
                       page_size);
  return hipGetLastError();
}

// One workgroup per row: X[row, :] (fp32) rounded to the storage type into
// taps[row, slot * H .. slot * H + H).
template <typename T>
__global__ __launch_bounds__(256) void tap_kernel(const float *X, int H, int slot, int n_slots, T *taps) {
  const int row = blockIdx.x;
  T *dst = taps + (size_t)row * n_slots * H + (size_t)slot * H;
  for (int i = threadIdx.x; i < H; i += blockDim.x) Storage<T>::store(dst, i, X[(size_t)row * H + i]);
}

hipError_t launch_tap(bool is_bf16, const float *X, int rows, int H, int slot, int n_slots, void *taps,
                      hipStream_t st) {
  if (is_bf16)
    hipLaunchKernelGGL(tap_kernel<bf16_t>, dim3(rows), dim3(256), 0, st, X, H, slot, n_slots, (bf16_t *)taps);
  else
    hipLaunchKernelGGL(tap_kernel<float>, dim3(rows), dim3(256), 0, st, X, H, slot, n_slots, (float *)taps);
  return hipGetLastError();
}

// Range check of device-resident indices (the compute kernels trust them).
// Blocks 0 .. batch-1: sequence s's context length, its block size and the page
// table entries its context and block cover; the remaining blocks: token ids
// and inject (seq, pos) pairs.  Every read is bounded by the sizes the host
// passes, whatever the values read; findings are OR-ed into *err.
__global__ __launch_bounds__(256) void check_inputs_kernel(CheckArgs a, int *err) {
  int bad = 0;
  const int s = blockIdx.x;
  if (s < a.batch) {
    const int ctx = a.ctx_len[s];
    if (ctx < 0 || ctx > a.max_ctx) bad |= kBadCtxLen;
    const long cap = (long)a.max_pages * a.page_size;
    if ((long)max(ctx, 0) + a.block_size > cap) bad |= kBadBlockPage;
    const long ctx_pages = ((long)max(ctx, 0) + a.page_size - 1) / a.page_size;
    const long all_pages = ((long)max(ctx, 0) + a.block_size + a.page_size - 1) / a.page_size;
    const int n_ctx = (int)min(ctx_pages, (long)a.max_pages), n_all = (int)min(all_pages, (long)a.max_pages);
    for (int i = threadIdx.x; i < n_all; i += blockDim.x) {
      const int pg = a.block_table[(size_t)s * a.max_pages + i];
      if (pg < 0 || pg >= a.n_pages) bad |= i < n_ctx ? kBadCtxPage : kBadBlockPage;
    }
    if (threadIdx.x == 0 && a.anchor && (a.anchor[s] < 0 || a.anchor[s] >= a.vocab)) bad |= kBadTokenId;
  } else {
    const int t0 = (s - a.batch) * blockDim.x + threadIdx.x, stride = (gridDim.x - a.batch) * blockDim.x;
    for (int t = t0; t < a.n_ids; t += stride)
      if (a.ids[t] < 0 || a.ids[t] >= a.vocab) bad |= kBadTokenId;
    for (int t = t0; t < a.n_new; t += stride) {
      const int q = a.seq[t], p = a.pos[t];
      if (q < 0 || q >= a.batch || p < 0 || (long)p >= (long)a.max_pages * a.page_size) {
        bad |= kBadInjectSlot;
      } else {
        const int pg = a.block_table[(size_t)q * a.max_pages + p / a.page_size];
        if (pg < 0 || pg >= a.n_pages) bad |= kBadInjectSlot;
      }
    }
  }
  if (bad) atomicOr(err, bad);
}

template <typename T>
static hipError_t launch_rmsnorm_t(const float *X, const T *gain, float eps, int rows, int H, int B, bool skip_anchor,
                                   T *Y, hipStream_t st) {
  const int n4 = H / 4, sa = skip_anchor ? 1 : 0;
  const dim3 grid(rows), block(kNormThreads);
  if (n4 <= 2 * kNormThreads) hipLaunchKernelGGL((rmsnorm_kernel<T, 2>), grid, block, 0, st, X, gain, eps, H, B, sa, Y);
  else if (n4 <= 4 * kNormThreads) hipLaunchKernelGGL((rmsnorm_kernel<T, 4>), grid, block, 0, st, X, gain, eps, H, B, sa, Y);
  else if (n4 <= 8 * kNormThreads) hipLaunchKernelGGL((rmsnorm_kernel<T, 8>), grid, block, 0, st, X, gain, eps, H, B, sa, Y);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_rmsnorm(bool is_bf16, const float *X, const void *gain, float eps, int rows, int H, int B,
                          bool skip_anchor, void *Y, hipStream_t st) {
  if (is_bf16) return launch_rmsnorm_t(X, (const bf16_t *)gain, eps, rows, H, B, skip_anchor, (bf16_t *)Y, st);
  return launch_rmsnorm_t(X, (const float *)gain, eps, rows, H, B, skip_anchor, (float *)Y, st);
}

hipError_t launch_argmax_reduce(const float *val, const int *idx, int rows, int n_groups, int *ids_out,
                                float *max_out, hipStream_t st) {
  hipLaunchKernelGGL(argmax_reduce_kernel, dim3(rows), dim3(256), 0, st, val, idx, n_groups, ids_out, max_out);
  return hipGetLastError();
}

hipError_t launch_accept(const int *draft, const int *target, int batch, int B, const int *block_len, int *tau,
                         int *bonus, hipStream_t st) {
  hipLaunchKernelGGL(accept_kernel, dim3(batch), dim3(64), 0, st, draft, target, B, block_len, tau, bonus);
  return hipGetLastError();
}

// Plain streaming read: each thread keeps 8 16-byte loads in flight per
// iteration (clamped addresses, out-of-range words masked), XOR-folds them and
// one lane per wave folds its wave's result into *sink.
constexpr int kReadThreads = 1024, kReadUnroll = 8;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4 *src, size_t n16, uint32_t *sink) {
  unsigned acc = 0;
  const size_t step = (size_t)gridDim.x * kReadThreads * kReadUnroll;
  for (size_t base = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < n16; base += step) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j) v[j] = src[min(base + (size_t)j * kReadThreads, n16 - 1)];
#pragma unroll
    for (int j = 0; j < kReadUnroll; ++j)
      if (base + (size_t)j * kReadThreads < n16) acc ^= v[j].x ^ v[j].y ^ v[j].z ^ v[j].w;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
  if ((threadIdx.x & 63) == 0) atomicXor(sink, acc);
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int n_cu, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + (size_t)kReadThreads * kReadUnroll - 1) / ((size_t)kReadThreads * kReadUnroll);
  if (blocks > (size_t)n_cu) blocks = n_cu;
  hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0, st, (const uint4 *)src, n16,
                     sink);
  return hipGetLastError();
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t st) {
  const size_t n16 = bytes / 16;
  if (n16 == 0) return hipSuccess;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(zero_kernel, dim3((unsigned)blocks), dim3(256), 0, st, (uint4 *)p, n16);
  return hipGetLastError();
}

hipError_t launch_check_inputs(const CheckArgs &a, int *err, hipStream_t st) {
  const int extra = (a.n_ids > 0 || a.n_new > 0) ? std::min(64, (std::max(a.n_ids, a.n_new) + 255) / 256) : 0;
  hipLaunchKernelGGL(check_inputs_kernel, dim3(a.batch + extra), dim3(256), 0, st, a, err);
  return hipGetLastError();
}

}  // namespace dflash
