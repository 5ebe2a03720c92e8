// Block attention of the drafter: the B block queries of every query head
// attend, without a mask, to the sequence's paged context keys plus the
// block's own B keys (in-block attention is non-causal).
//
// Work items are (sequence, context chunk, KV head): the G = nq/nkv query heads
// of one KV head share every K/V byte, so an item streams its chunk of K/V once
// for G*B query rows.  Items write an unnormalised partial (O, running max,
// running sum); a merge kernel combines the chunks of a (sequence, KV head) in
// chunk order.
//
// Inside an item, 64-key sub-blocks of K and V are staged in LDS (V
// transposed).  Scores are formed as S^T = K Q^T on the matrix cores, so a
// lane holds 4 keys of one query row; the exponentiated scores of two 16-key
// tiles are then exactly that lane's fragment of P^T, and O^T = V^T P^T keeps
// the query row in the same lane, which makes the online-softmax rescale
// lane-local.  With bf16 storage the softmax weights enter the P*V product as
// two bf16 terms (P_hi + P_lo), so P keeps about 16 mantissa bits.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kSub = 64;        // keys per LDS sub-block
constexpr float kTau = 8.0f;    // log2 headroom of the lazy softmax rescale
constexpr int kPage = 16;       // keys per cache page (the only page size accepted)
constexpr float kLog2e = 1.4426950408889634f;

int attn_chunk(int batch, int max_ctx, int block_size, int nq, int nkv, int cu) {
  // aim for a few items per compute unit; chunk in [64, 512] keys, multiple of 64
  const long keys = (long)batch * (max_ctx + block_size) * nkv;
  long c = keys / 1024;
  c = (c + kSub - 1) / kSub * kSub;
  if (c < kSub) c = kSub;
  if (c > 512) c = 512;
  // Items run in rounds of the resident workgroups (4 per compute unit for up
  // to 64 block queries per KV head, 2 for up to 128).  When a chunk at most
  // three times as long puts every item in one round, take the shortest such chunk:
  // a last round with a few items costs a whole item time (with the declared
  // maximum context as every sequence's length).
  const long slots = (long)cu * ((nq / nkv) * block_size <= 64 ? 4 : 2);
  auto items = [&](long ch) { return (long)batch * ((max_ctx + block_size + ch - 1) / ch) * nkv; };
  if (items(c) > slots) {
    for (long c1 = c + kSub; c1 <= 3 * c && c1 <= 1024; c1 += kSub)
      if (items(c1) <= slots) return (int)c1;
  }
  return (int)c;
}

int attn_max_items(int batch, int max_ctx, int block_size, int nkv, int chunk) {
  return batch * ((max_ctx + block_size + chunk - 1) / chunk) * nkv;
}

// Context keys a sequence attends to: all ctx of them, or with a sliding
// window the last `window` (the block keys always).
__device__ __forceinline__ int attended_ctx(int ctx, int window) { return window > 0 ? min(ctx, window) : ctx; }

// Locate flat chunk index f among the sequences (chunks per sequence =
// ceil((attended context + B) / chunk)).  Executed by one wave; returns seq
// (-1 when f is beyond the total) and the sequence's first flat chunk index.
__device__ void find_seq(const int *ctx_len, int window, int batch, int B, int chunk, int f, int *seq_out,
                         int *first_out) {
  const int lane = threadIdx.x & 63;
  int base = 0;
  for (int s0 = 0; s0 < batch; s0 += 64) {
    const int s = s0 + lane;
    const int n = s < batch ? (attended_ctx(ctx_len[s], window) + B + chunk - 1) / chunk : 0;
    int inc = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int t = __shfl_up(inc, o);
      if (lane >= o) inc += t;
    }
    const int excl = base + inc - n;
    const bool hit = s < batch && f >= excl && f < excl + n;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      *seq_out = __shfl(s, src);
      *first_out = __shfl(excl, src);
      return;
    }
    base += __shfl(inc, 63);
  }
  *seq_out = -1;
  *first_out = 0;
}

// NW waves per workgroup, one per 16-row tile of the G*B block queries (4 for
// G*B <= 64, 8 for G*B <= 128); the first 256 threads stage K and V.  One tile
// per wave keeps the register footprint small enough for 16 waves per CU.
template <typename T, int HD, int NW>
// Four waves per SIMD (the second bound counts waves per execution unit): four
// 4-wave or two 8-wave workgroups per compute unit, at most 128 VGPRs.
__global__ __launch_bounds__(NW * 64, 4) void attn_partial_kernel(const AttnArgs a) {
  constexpr int NT = NW * 64;
  constexpr int EPV = 16 / (int)sizeof(T);      // elements per 16-byte vector
  constexpr int VPK = HD / EPV;                 // vectors per key row
  constexpr int KSTR = HD + EPV;                // LDS row stride of K (elements)
  // LDS row stride of V^T (elements), padded: row r starts 4 (r % 8) dwords
  // into the banks.  bf16 rows also XOR their 16-byte chunk index (8 keys)
  // with (r / 8) % 8.  A V thread writes one chunk of rows dg*8 + e, so without
  // it the 16 lanes of a key group (rows 8 apart, the same r % 8) all hit the
  // same banks (16-way conflicts); with it they take 8 positions (2-way), and
  // the fragment reads of 16 consecutive rows stay within 2 ways.
  constexpr int VSTR = kSub + EPV;
  auto vt_chunk = [](int row, int c) { return sizeof(T) == 2 ? c ^ ((row >> 3) & 7) : c; };
  constexpr int NU = HD / 32;                   // k-chunks over head_dim
  constexpr int ND = HD / 16;                   // d tiles
  __shared__ __align__(16) T k_lds[kSub * KSTR];
  __shared__ __align__(16) T vt_lds[HD * VSTR];
  __shared__ int s_seq, s_first;
  __shared__ int s_pages[1024 / 16 + 1];          // page ids of this item's context keys

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g4 = lane >> 4, ln = lane & 15;
  const int item = blockIdx.x;
  const int f = item / a.nkv, g = item % a.nkv;
  // One sequence and no sliding window: item f is chunk f of sequence 0, so
  // its page-table entries are requested together with the context length and
  // the query fragments (one round trip) instead of after a lookup of the
  // item's sequence (three round trips; 1 us per launch, measured).
  const bool single = a.batch == 1 && a.window == 0;
  int spec_page = 0;
  if (single && tid <= a.chunk / kPage)
    spec_page = a.block_table[min((f * a.chunk) / kPage + tid, a.max_pages - 1)];
  if (!single) {
    if (wave == 0) {
      int sq, first;
      find_seq(a.ctx_len, a.window, a.batch, a.block_size, a.chunk, f, &sq, &first);
      if (lane == 0) { s_seq = sq; s_first = first; }
    }
    __syncthreads();
    if (s_seq < 0) return;
  }
  const int s = single ? 0 : s_seq;
  const int c = single ? f : f - s_first;
  const int B = a.block_size, G = a.nq / a.nkv, GB = G * B;
  const int ctx = a.ctx_len[s];
  if (single && f * a.chunk >= ctx + B) return;   // past the sequence's chunks (uniform)
  // block keys this sequence attends to (a per-sequence block size): the
  // attended keys stay one contiguous range, so a smaller block only ends it
  // earlier (a chunk past the end is empty and its partial carries no weight)
  const int bs = a.block_len ? min(max(a.block_len[s], 1), a.block_size) : a.block_size;
  // keys k0 .. ctx - 1 of the context (k0 > 0 under a sliding window), then the block
  const int kbeg = (ctx - attended_ctx(ctx, a.window)) + c * a.chunk;
  const int kend = min(kbeg + a.chunk, ctx + bs);
  const int MTQ = (GB + 15) / 16;
  const T *Q = (const T *)a.q;
  const T *Kc = (const T *)a.kc, *Vc = (const T *)a.vc, *Kb = (const T *)a.kb, *Vb = (const T *)a.vb;
  const float scale = kLog2e / sqrtf((float)HD);
  const float mask_raw = -1e30f / scale;        // a masked key's raw score: -1e30 once scaled

  // query fragments of this wave's tiles (B operand: column = query row)
  Frag<T> qf[1][NU];
  bool tile_on[1];
  int qrow_j[1];   // block position of this lane's query row
#pragma unroll
  for (int t = 0; t < 1; ++t) {
    const int qt = wave;
    tile_on[t] = qt < MTQ;
    const int r = qt * 16 + ln;
    const bool ok = tile_on[t] && r < GB;
    const int hh = ok ? r / B : 0, j = ok ? r % B : 0;
    qrow_j[t] = j;
    const T *qp = Q + ((size_t)(s * B + j) * a.nq + g * G + hh) * HD + 8 * g4;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      if (ok) qf[t][u].load(qp + 32 * u); else qf[t][u].zero();
    }
  }
  f32x4 o[1][ND];
  float m_run[1], l_run[1];
#pragma unroll
  for (int t = 0; t < 1; ++t) {
    m_run[t] = -1e30f;
    l_run[t] = 0.f;
#pragma unroll
    for (int d = 0; d < ND; ++d) o[t][d] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Sub-block staging.  bf16: threads 0..127 each carry 8 16-byte chunks of K
  // (straight rows); threads 128..255 each carry an 8-key x 8-dim block of V,
  // transposed in registers and written as 8 rows of V^T.  The next sub-block's
  // chunks are loaded while the current one is processed.  fp32 (small head
  // dims only) stages element by element.
  uint4 pre[8];
  // page ids of the item's context keys, read once (a dependent global load per
  // key would serialise every in-flight K/V load behind it)
  const int p0 = kbeg / kPage;
  if (single) {
    if (tid <= a.chunk / kPage) s_pages[tid] = spec_page;   // entries past the context are never read
  } else {
    for (int i = tid; i <= (min(kend, ctx) - 1) / kPage - p0 && kbeg < ctx; i += NT)
      s_pages[i] = a.block_table[(size_t)s * a.max_pages + p0 + i];
  }
  __syncthreads();
  auto key_ptr = [&](int t, const T *ctxp, const T *blkp) -> const T * {
    if (t < ctx) {
      const int page = s_pages[t / kPage - p0];
      return ctxp + (((size_t)page * kPage + t % kPage) * a.nkv + g) * HD;
    }
    return blkp + ((size_t)(s * B + (t - ctx)) * a.nkv + g) * HD;
  };
  // Fast path for a sub-block of context keys only, starting on a page
  // boundary (every sub-block of a sequence but the last without a sliding
  // window): a K thread's load j reads key tid/VPK + KPP*j, so its page is
  // the same for the whole wave (read once, kept scalar) and its slot is
  // tid/VPK + (KPP*j) % 16; a V thread's 8 consecutive keys share one page.
  // Addresses are a base plus a 32-bit byte offset whose per-lane part is
  // fixed before the loop: the K base is wave-uniform (page and slot), the V
  // offset holds the lane's page too (a cache layer under 4 GB).
  constexpr int KPP = 128 / VPK;                // keys per pass of the K threads
  const unsigned slot_b = (unsigned)(a.nkv * HD * (int)sizeof(T));   // bytes per cache slot
  const unsigned page_b = slot_b * kPage;
  const int u128 = tid & 127, v_kg = u128 / (HD / 8);
  // per-lane byte offset: K threads key slot tid/VPK, piece tid%VPK; V threads
  // slot (kg%2)*8 of their 8-key group, dims dg*8..
  const unsigned lane_b =
      (unsigned)sizeof(T) * (tid < 128 ? (unsigned)((u128 / VPK) * (a.nkv * HD) + g * HD + (u128 % VPK) * EPV)
                                       : (unsigned)(((v_kg & 1) * 8) * (a.nkv * HD) + g * HD + (u128 % (HD / 8)) * 8));
  // waves 0, 1 stage K and waves 2, 3 stage V: a test the compiler knows is
  // wave-uniform
  const int wave_u = __builtin_amdgcn_readfirstlane(tid >> 6);
  // The fast path's page lookups for the next sub-block are read from LDS
  // before this sub-block's LDS writes are issued: LDS operations complete in
  // order, so a lookup queued behind the eight 16-byte writes waited for all
  // of them.  K's four pages are wave-uniform, V keeps its byte offset.
  struct FastPages {
    int k[4];
    unsigned vo;
  };
  auto fetch_fast = [&](int sub) {
    FastPages f{{0, 0, 0, 0}, 0u};
    const int pq = sub / kPage - p0;
    if (wave_u < 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) f.k[q] = __builtin_amdgcn_readfirstlane(s_pages[pq + q]);
    } else if (v_kg * 8 < kSub) {
      int t_ = tid;
      asm volatile("" : "+v"(t_));
      f.vo = (unsigned)s_pages[pq + ((t_ & 127) / (HD / 8)) / 2] * page_b + lane_b;
    }
    return f;
  };
  auto load_sub_fast2 = [&](const FastPages &f) {
    if (wave_u < 2) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        if (128 * j + tid >= kSub * VPK) break;   // never for HD = 128; HD = 64 stops at 4
        const char *pb = reinterpret_cast<const char *>(Kc) + (size_t)f.k[(KPP * j) / kPage] * page_b +
                         ((KPP * j) % kPage) * slot_b;
        pre[j] = *reinterpret_cast<const uint4 *>(pb + lane_b);
      }
    } else if (v_kg * 8 < kSub) {
#pragma unroll
      for (int j = 0; j < 8; ++j)
        pre[j] = *reinterpret_cast<const uint4 *>(reinterpret_cast<const char *>(Vc) + (f.vo + j * slot_b));
    }
  };
  auto fast_ok = [&](int sub) { return a.off32 && sub % kPage == 0 && sub + kSub <= min(ctx, kend); };
  FastPages fp{{0, 0, 0, 0}, 0u};
  auto load_sub = [&](int sub) {
    if (tid >= 256) return;
    if constexpr (sizeof(T) == 2) {
      if (fast_ok(sub)) {   // uniform
        load_sub_fast2(fp);
        return;
      }
      if (tid < 128) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = tid + 128 * j, kk = i / VPK, vv = i % VPK, t = sub + kk;
          pre[j] = (i < kSub * VPK && t < kend) ? *reinterpret_cast<const uint4 *>(key_ptr(t, Kc, Kb) + vv * EPV)
                                                 : make_uint4(0, 0, 0, 0);
        }
      } else {
        const int u = tid - 128, kg = u / (HD / 8), dg = u % (HD / 8);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int t = sub + kg * 8 + j;
          pre[j] = (kg * 8 < kSub && t < kend) ? *reinterpret_cast<const uint4 *>(key_ptr(t, Vc, Vb) + dg * 8)
                                                : make_uint4(0, 0, 0, 0);
        }
      }
    }
  };
  auto store_sub = [&](int sub) {
    if (tid >= 256) return;
    if constexpr (sizeof(T) == 2) {
      if (tid < 128) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = tid + 128 * j, kk = i / VPK, vv = i % VPK;
          if (i < kSub * VPK) *reinterpret_cast<uint4 *>(k_lds + kk * KSTR + vv * EPV) = pre[j];
        }
      } else {
        const int u = tid - 128, kg = u / (HD / 8), dg = u % (HD / 8);
        if (kg * 8 < kSub) {
          // pre[j] holds dims dg*8..+7 of key kg*8+j; row e of V^T gets key j's
          // dim e: word m of the row = (key 2m, key 2m+1), one byte permute each
          const uint32_t *w = reinterpret_cast<const uint32_t *>(pre);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            uint32_t o[4];
#pragma unroll
            for (int m = 0; m < 4; ++m)
              o[m] = __builtin_amdgcn_perm(w[(2 * m + 1) * 4 + e / 2], w[(2 * m) * 4 + e / 2],
                                           (e & 1) ? 0x07060302u : 0x05040100u);
            const int row = dg * 8 + e;
            *reinterpret_cast<uint4 *>(vt_lds + row * VSTR + vt_chunk(row, kg) * 8) = make_uint4(o[0], o[1], o[2], o[3]);
          }
        }
      }
    } else {
      for (int i = tid; i < kSub * VPK; i += 256) {
        const int kk = i / VPK, vv = i - kk * VPK;
        const int t = sub + kk;
        uint4 kx = make_uint4(0, 0, 0, 0), vx = make_uint4(0, 0, 0, 0);
        if (t < kend) {
          kx = *reinterpret_cast<const uint4 *>(key_ptr(t, Kc, Kb) + vv * EPV);
          vx = *reinterpret_cast<const uint4 *>(key_ptr(t, Vc, Vb) + vv * EPV);
        }
        *reinterpret_cast<uint4 *>(k_lds + kk * KSTR + vv * EPV) = kx;
        const T *ve = reinterpret_cast<const T *>(&vx);
#pragma unroll
        for (int e = 0; e < EPV; ++e) vt_lds[(vv * EPV + e) * VSTR + kk] = ve[e];
      }
    }
  };

  if (sizeof(T) == 2 && fast_ok(kbeg) && wave_u < 4) fp = fetch_fast(kbeg);
  load_sub(kbeg);
  for (int sub = kbeg; sub < kend; sub += kSub) {
    lds_barrier();
    if (sizeof(T) == 2 && sub + kSub < kend && fast_ok(sub + kSub) && wave_u < 4) fp = fetch_fast(sub + kSub);
    store_sub(sub);
    if (sub + kSub < kend) load_sub(sub + kSub);
    lds_barrier();
#pragma unroll
    for (int kb2 = 0; kb2 < kSub; kb2 += 32) {
      if (sub + kb2 >= kend) break;
      // V^T fragments for all d tiles (A operand: row = d, k = keys)
#pragma unroll
      for (int t = 0; t < 1; ++t) {
        if (!tile_on[t]) continue;
        // S^T = K Q^T for two 16-key tiles; each K fragment is read one
        // product ahead of its use
        f32x4 st[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
        auto read_kf = [&](int q) {
          Frag<T> kf;
          kf.load(k_lds + (kb2 + (q / NU) * 16 + ln) * KSTR + 8 * g4 + 32 * (q % NU));
          return kf;
        };
        Frag<T> kcur = read_kf(0);
#pragma unroll
        for (int q = 0; q < 2 * NU; ++q) {
          const Frag<T> knext = read_kf(q + 1 < 2 * NU ? q + 1 : q);
          st[q / NU] = mma(st[q / NU], kcur, qf[t][q % NU]);
          kcur = knext;
        }
        // raw scores; a masked key gets -1e30 / scale, i.e. -1e30 once scaled.
        // When every key of this half is visible to every row (uniform) the
        // per-key mask is skipped.  The scale folds into the exponent's FMA.
        float p[8];
        if (!a.causal && sub + kb2 + 32 <= kend) {
#pragma unroll
          for (int e = 0; e < 8; ++e) p[e] = f4get(st[e / 4], e % 4);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int key = sub + kb2 + (e / 4) * 16 + 4 * g4 + e % 4;
            // causal (target verify): block row j sees keys up to position ctx + j
            const bool vis = key < kend && (!a.causal || key <= ctx + qrow_j[t]);
            p[e] = vis ? f4get(st[e / 4], e % 4) : mask_raw;
          }
        }
        // scale > 0: the max of the scaled scores, exactly
        float bmax = fmaxf(fmaxf(fmaxf(p[0], p[1]), fmaxf(p[2], p[3])), fmaxf(fmaxf(p[4], p[5]), fmaxf(p[6], p[7]))) * scale;
        bmax = fmaxf(bmax, __shfl_xor(bmax, 16));
        bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
        // Lazy rescale: the running reference m_run moves (and O, l are
        // rescaled) only when some row's new maximum exceeds it by more than
        // kTau; otherwise weights up to 2^kTau enter as they are.  O / l and
        // the chunk merge do not depend on the reference, so the result is the
        // same up to rounding, and the rescale becomes a rare uniform branch.
        if (__any(bmax > m_run[t] + kTau)) {
          const float m_new = fmaxf(m_run[t], bmax);
          // arguments are <= 0; the bare hardware exp2 (no denormal-range
          // fix-up: weights below 2^-126 of the reference count as 0)
          const float alpha = __builtin_amdgcn_exp2f(m_run[t] - m_new);
          l_run[t] *= alpha;
#pragma unroll
          for (int d = 0; d < ND; ++d) o[t][d] *= alpha;
          m_run[t] = m_new;
        }
        const float mr = m_run[t];
        float psum = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          p[e] = __builtin_amdgcn_exp2f(fmaf(p[e], scale, -mr));
          psum += p[e];
        }
        l_run[t] += psum;
        // bf16: P = P_hi + P_lo, two bf16 terms, so the product keeps ~16
        // mantissa bits of the softmax weights instead of 8
        Frag<T> pf, pf_lo;
        pf.set(p);
        if constexpr (sizeof(T) == 2) {
          float lo[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) lo[e] = p[e] - pf.get(e);
          pf_lo.set(lo);
        }
        // V^T fragment of d tile d (A operand: row = d, k = keys)
        auto read_vf = [&](int d) {
          Frag<T> vf;
          if constexpr (sizeof(T) == 2) {
            // keys k0 .. k0+3 (chunk k0/8) and k0+16 .. (chunk k0/8 + 2) of V^T
            // row d*16 + ln.  The chunk bits (kb2/8: bit 2; g4/2: bit 0; +2:
            // bit 1) and the swizzle ((2d + ln/8) % 8: bits 1-2 and bit 0) are
            // disjoint, so the swizzled chunk is a compile-time part XOR the
            // lane's bit (g4/2 ^ ln/8): one lane base and immediate offsets.
            const T *vrow = vt_lds + ln * VSTR + 4 * (g4 & 1) + 8 * ((g4 >> 1) ^ (ln >> 3)) + d * 16 * VSTR;
            const uint2 lo = *reinterpret_cast<const uint2 *>(vrow + 8 * ((kb2 >> 3) ^ ((2 * d) & 7)));
            const uint2 hi = *reinterpret_cast<const uint2 *>(vrow + 8 * ((kb2 >> 3) ^ ((2 * d) & 7) ^ 2));
            reinterpret_cast<Frag<bf16_t> &>(vf).v = make_uint4(lo.x, lo.y, hi.x, hi.y);
          } else {
            const T *vr = vt_lds + (d * 16 + ln) * VSTR + kb2 + 4 * g4;
            const float4 lo = *reinterpret_cast<const float4 *>(vr);
            const float4 hi = *reinterpret_cast<const float4 *>(vr + 16);
            reinterpret_cast<Frag<float> &>(vf).v = f32x8{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
          }
          return vf;
        };
        // one fragment of lookahead: tile d+1 is read before tile d's products
        Frag<T> vcur = read_vf(0);
#pragma unroll
        for (int d = 0; d < ND; ++d) {
          const Frag<T> vnext = read_vf(d + 1 < ND ? d + 1 : d);
          o[t][d] = mma(o[t][d], vcur, pf);
          if constexpr (sizeof(T) == 2) o[t][d] = mma(o[t][d], vcur, pf_lo);
          vcur = vnext;
        }
      }
    }
  }

  // partial results: O^T (lane: query row ln, d rows 4*g4..), max, sum
  const int GBP = MTQ * 16;
#pragma unroll
  for (int t = 0; t < 1; ++t) {
    if (!tile_on[t]) continue;
    float l = l_run[t];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    const int r = wave * 16 + ln;
    if (r >= GB) continue;
    float *po = a.partial + ((size_t)item * GBP + r) * HD;
#pragma unroll
    for (int d = 0; d < ND; ++d)
#pragma unroll
      for (int i = 0; i < 4; ++i) po[d * 16 + 4 * g4 + i] = f4get(o[t][d], i);
    if (g4 == 0) {
      a.stats[((size_t)item * GBP + r) * 2 + 0] = m_run[t];
      a.stats[((size_t)item * GBP + r) * 2 + 1] = l;
    }
  }
}

// One wave per (sequence, KV head, query row): combine the chunk partials.
// Lanes fetch the chunks' (max, sum) statistics in parallel; the weighted sum
// of the partial outputs then runs over chunks with the loads of DEPTH chunks
// in flight at once, in chunk order (deterministic).  DEPTH is sized to the
// most chunks a sequence can have, so short chunk lists do not re-read.
template <typename T, int HD, int DEPTH>
__global__ __launch_bounds__(64) void attn_merge_kernel(const AttnArgs a) {
  const int lane = threadIdx.x;
  const int B = a.block_size, G = a.nq / a.nkv, GB = G * B;
  const int MTQ = (GB + 15) / 16, GBP = MTQ * 16;
  const int r = blockIdx.x % GB;
  const int sg = blockIdx.x / GB;
  const int s = sg / a.nkv, g = sg % a.nkv;
  // first flat chunk of sequence s (prefix over the ragged chunk counts)
  int base = 0;
  for (int s0 = 0; s0 < s; s0 += 64) {
    const int q = s0 + lane;
    int n = q < s ? (attended_ctx(a.ctx_len[q], a.window) + B + a.chunk - 1) / a.chunk : 0;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) n += __shfl_xor(n, o);
    base += n;
  }
  int nch = (attended_ctx(a.ctx_len[s], a.window) + B + a.chunk - 1) / a.chunk;
  // chunks past the launched item range were never computed (ctx_len above the
  // declared maximum); never read beyond the partial buffers
  if ((base + nch) * a.nkv > a.max_items) nch = max(0, a.max_items / a.nkv - base);
  auto stat = [&](int c, int k) { return a.stats[(((size_t)(base + c) * a.nkv + g) * GBP + r) * 2 + k]; };
  // global max over chunks, then the normaliser
  float M = -1e30f;
  for (int c = lane; c < nch; c += 64) M = fmaxf(M, stat(c, 0));
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) M = fmaxf(M, __shfl_xor(M, o));
  float lsum = 0.f;
  for (int c = lane; c < nch; c += 64) lsum += exp2f(stat(c, 0) - M) * stat(c, 1);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) lsum += __shfl_xor(lsum, o);
  constexpr int PER = HD / 64;
  float acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = 0.f;
  for (int c0 = 0; c0 < nch; c0 += DEPTH) {
    // weight of chunk c0 + lane, broadcast below
    const float wl = c0 + lane < nch ? exp2f(stat(c0 + lane, 0) - M) : 0.f;
    const int cn = min(DEPTH, nch - c0);
    // DEPTH chunks' partial outputs in flight at once; past cn the last valid
    // chunk is re-read (a cache hit) and weighted 0
    float po[DEPTH][PER];
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const float *p = a.partial + (((size_t)(base + c0 + min(j, cn - 1)) * a.nkv + g) * GBP + r) * HD;
#pragma unroll
      for (int e = 0; e < PER; ++e) po[j][e] = p[lane + 64 * e];
    }
#pragma unroll
    for (int j = 0; j < DEPTH; ++j) {
      const float w = j < cn ? __shfl(wl, j) : 0.f;
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] += w * po[j][e];
    }
  }
  const float inv = lsum > 0.f ? 1.0f / lsum : 0.f;
  const int hh = r / B, j = r % B;
  T *O = (T *)a.o;
  const size_t ob = ((size_t)(s * B + j) * a.nq + g * G + hh) * HD;
#pragma unroll
  for (int e = 0; e < PER; ++e) Storage<T>::store(O, ob + lane + 64 * e, acc[e] * inv);
}

// One sequence: a workgroup of four waves per (KV head, query row).  Wave w
// combines chunks w, w + 4, .. (at most DW of them), each lane holding HD/64
// consecutive head dims.  The number of chunks the partial launch computed is
// known without the context length, so the statistics and partial outputs of
// all of them are requested at once, with the context length (one round trip;
// chunks past the sequence's own count are masked after it arrives).  The four
// waves' (max, sum, weighted output) states are combined in LDS in wave order
// (deterministic).
template <typename T, int HD, int DW>
__global__ __launch_bounds__(256) void attn_merge1_kernel(const AttnArgs a) {
  constexpr int PER = HD / 64;
  __shared__ float s_m[4], s_l[4];
  __shared__ float s_o[4][HD];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = a.block_size, G = a.nq / a.nkv, GB = G * B;
  const int GBP = (GB + 15) / 16 * 16;
  const int r = blockIdx.x % GB, g = blockIdx.x / GB;
  const int nl = a.max_items / a.nkv;                  // chunks launched (>= the sequence's)
  const int ctx = a.ctx_len[0];
  float2 st[DW];
  float po[DW][PER];
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    const int cc = min(wave + 4 * j, nl - 1);
    const size_t it = (size_t)cc * a.nkv + g;
    st[j] = *reinterpret_cast<const float2 *>(a.stats + (it * GBP + r) * 2);
    const float *pp = a.partial + (it * GBP + r) * HD + PER * lane;
#pragma unroll
    for (int e = 0; e < PER; ++e) po[j][e] = pp[e];
  }
  const int nch = min(nl, (attended_ctx(ctx, a.window) + B + a.chunk - 1) / a.chunk);
  float m = -1e30f;
#pragma unroll
  for (int j = 0; j < DW; ++j)
    if (wave + 4 * j < nch) m = fmaxf(m, st[j].x);
  float l = 0.f, o[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) o[e] = 0.f;
#pragma unroll
  for (int j = 0; j < DW; ++j) {
    const bool live = wave + 4 * j < nch;
    const float wgt = live ? exp2f(st[j].x - m) : 0.f;
    l += live ? wgt * st[j].y : 0.f;
#pragma unroll
    for (int e = 0; e < PER; ++e) o[e] += live ? wgt * po[j][e] : 0.f;
  }
  if (lane == 0) { s_m[wave] = m; s_l[wave] = l; }
#pragma unroll
  for (int e = 0; e < PER; ++e) s_o[wave][PER * lane + e] = o[e];
  __syncthreads();
  if (tid < HD) {
    const float M = fmaxf(fmaxf(s_m[0], s_m[1]), fmaxf(s_m[2], s_m[3]));
    float L = 0.f, v = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2f(s_m[w] - M);
      L += sc * s_l[w];
      v += sc * s_o[w][tid];
    }
    const int hh = r / B, jb = r % B;
    T *O = (T *)a.o;
    Storage<T>::store(O, ((size_t)jb * a.nq + g * G + hh) * HD + tid, L > 0.f ? v / L : 0.f);
  }
}

template <typename T, int HD>
static hipError_t launch_attn_t(const AttnArgs &a, hipStream_t st) {
  const int GBq = (a.nq / a.nkv) * a.block_size;
  if (GBq <= 64) hipLaunchKernelGGL((attn_partial_kernel<T, HD, 4>), dim3(a.max_items), dim3(256), 0, st, a);
  else hipLaunchKernelGGL((attn_partial_kernel<T, HD, 8>), dim3(a.max_items), dim3(512), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int GB = (a.nq / a.nkv) * a.block_size;
  const int max_chunks = a.max_items / (a.batch * a.nkv);
  if (a.batch == 1 && max_chunks <= 64) {
    const dim3 grid(a.nkv * GB), block(256);
    if (max_chunks <= 16) hipLaunchKernelGGL((attn_merge1_kernel<T, HD, 4>), grid, block, 0, st, a);
    else if (max_chunks <= 32) hipLaunchKernelGGL((attn_merge1_kernel<T, HD, 8>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_merge1_kernel<T, HD, 16>), grid, block, 0, st, a);
  } else if (max_chunks <= 16)
    hipLaunchKernelGGL((attn_merge_kernel<T, HD, 16>), dim3(a.batch * a.nkv * GB), dim3(64), 0, st, a);
  else
    hipLaunchKernelGGL((attn_merge_kernel<T, HD, 64>), dim3(a.batch * a.nkv * GB), dim3(64), 0, st, a);
  return hipGetLastError();
}

hipError_t launch_attention(bool is_bf16, const AttnArgs &a, hipStream_t st) {
  if (is_bf16) return a.hd == 128 ? launch_attn_t<bf16_t, 128>(a, st) : launch_attn_t<bf16_t, 64>(a, st);
  return a.hd == 128 ? launch_attn_t<float, 128>(a, st) : launch_attn_t<float, 64>(a, st);
}

}  // namespace dflash
