// Weight-streaming matrix-core GEMM for few rows (the drafter's projections at
// small batch) with fused epilogues.
//
// out[M, N] = A[M, K] * W[N, K]^T, W row-major [out, in] as stored.
//
// Work decomposition.  A workgroup owns one 16-column tile and up to 64 rows
// and runs the whole K: its 8 waves take interleaved blocks of 32-wide
// k-chunks, and their partial tiles are summed through LDS in wave order
// (deterministic, no cross-workgroup traffic, no device-scope fences).  Weights
// stream from HBM straight into matrix-core fragments; the activations (tiny,
// L2-resident) are read into fragments the same way.
//
// Column maps.  The 16 columns of a tile are mapped to weight rows so that an
// epilogue's operands sit in the same tile:
//   RoPE (q/k/v, injected k/v): 8 rotation pairs (i, i + d/2) of one head,
//   SwiGLU: 8 gate rows beside their 8 up rows,
//   otherwise 16 consecutive rows.
#include "dflash_device.h"
#include "dflash_internal.h"

namespace dflash {

constexpr int kGemmWaves = 8;

int gemm_rows_per_group(int M) { return M <= 16 ? 16 : (M <= 32 ? 32 : 64); }

int gemm_tiles(Epilogue epi, int N, int ffn) { return epi == EPI_SWIGLU ? ffn / 8 : N / 16; }

// Weight row (= output feature) of column c of tile t.
template <int EPI>
__device__ __forceinline__ int weight_row(const GemmArgs &a, int t, int c) {
  if constexpr (EPI == EPI_SWIGLU) {
    return c < 8 ? t * 8 + c : a.ffn + t * 8 + (c - 8);
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int tph = a.hd / 16;                       // tiles per head
    const int h = t / tph, j0 = (t - h * tph) * 8;
    return h * a.hd + (c < 8 ? j0 + c : a.hd / 2 + j0 + (c - 8));
  } else {
    return t * 16 + c;
  }
}

template <typename T, int EPI>
__device__ void gemm_epilogue(const GemmArgs &a, const float *ct, int MP, int row0, int t, int layer) {
  // ct: [MP][16] fp32 tile, row-major
  const int tid = threadIdx.x;
  if constexpr (EPI == EPI_STORE || EPI == EPI_STORE_F32 || EPI == EPI_RESID) {
    for (int i = tid; i < MP * 16; i += blockDim.x) {
      const int r = i >> 4, c = i & 15, row = row0 + r;
      if (row >= a.M) continue;
      const int n = t * 16 + c;
      const float v = ct[i];
      if constexpr (EPI == EPI_STORE) Storage<T>::store((T *)a.out, (size_t)row * a.ldo + n, v);
      else if constexpr (EPI == EPI_STORE_F32) ((float *)a.out)[(size_t)row * a.ldo + n] = v;
      else a.X[(size_t)row * a.ldx + n] += v;
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    for (int i = tid; i < MP * 8; i += blockDim.x) {
      const int r = i >> 3, c = i & 7, row = row0 + r;
      if (row >= a.M) continue;
      const float gt = ct[r * 16 + c], up = ct[r * 16 + 8 + c];
      Storage<T>::store((T *)a.out, (size_t)row * a.ldo + t * 8 + c, silu_mul(gt, up));
    }
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_INJECT) {
    const int hd = a.hd, half = hd / 2;
    const int qcols = (EPI == EPI_QKV) ? a.nq * hd : 0;
    const int kcols = a.nkv * hd;
    const int tph = hd / 16;
    const int j0 = (t % tph) * 8;
    for (int i = tid; i < MP * 8; i += blockDim.x) {
      const int r = i >> 3, c = i & 7, row = row0 + r;
      if (row >= a.M) continue;
      const int n = weight_row<EPI>(a, t, c);       // lower element of the pair
      const float x1 = ct[r * 16 + c], x2 = ct[r * 16 + 8 + c];
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
        rope_cs_inv(pos, rope_inv_freq(j0 + c, hd, a.log2_theta), &cs, &sn);
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
    // one thread per row: maximum of the 16 columns, lowest column on ties (a
    // NaN never wins; no number above -inf leaves the first column)
    for (int r = tid; r < MP; r += blockDim.x) {
      const int row = row0 + r;
      if (row >= a.M) continue;
      float best = -INFINITY;
      int bc = 0;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        const float v = ct[r * 16 + c];
        if (v > best) { best = v; bc = c; }
      }
      a.amax_val[(size_t)row * a.n_groups + t] = best;
      a.amax_idx[(size_t)row * a.n_groups + t] = t * 16 + bc;
    }
  }
}

template <typename T, int MT, int EPI>
__global__ __launch_bounds__(kGemmWaves * 64) void gemm_kernel(const GemmArgs a) {
  constexpr int MP = 16 * MT;
  constexpr int U = MT == 1 ? 8 : (MT == 2 ? 4 : 2);   // k-chunks per batch of loads
  __shared__ float red[kGemmWaves][MP * 16];
  __shared__ float ct[MP * 16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, g = lane >> 4, ln = lane & 15;
  const int t = blockIdx.x;
  const int layer = blockIdx.y / a.m_groups, mg = blockIdx.y - layer * a.m_groups;
  const int row0 = mg * MP;
  const T *A = (const T *)a.A;
  const T *W = (const T *)a.W[layer];
  const T *wp = W + (size_t)weight_row<EPI>(a, t, ln) * a.ldw + 8 * g;
  const T *ap[MT];
  bool aok[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = row0 + mt * 16 + ln;
    aok[mt] = row < a.M;
    ap[mt] = A + (size_t)(aok[mt] ? row : 0) * a.lda + 8 * g;
  }

  f32x4 acc[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) acc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nchunk = a.K / 32;
  const int nblk = (nchunk + U - 1) / U;
  for (int blk = wave; blk < nblk; blk += kGemmWaves) {
    const int c0 = blk * U;
    if (c0 + U <= nchunk) {
      Frag<T> wf[U], af[MT][U];
#pragma unroll
      for (int j = 0; j < U; ++j) wf[j].load(wp + 32 * (c0 + j));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int j = 0; j < U; ++j) {
          if (aok[mt]) af[mt][j].load(ap[mt] + 32 * (c0 + j)); else af[mt][j].zero();
        }
#pragma unroll
      for (int j = 0; j < U; ++j)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) acc[mt] = mma(acc[mt], af[mt][j], wf[j]);
    } else {
      for (int c = c0; c < nchunk; ++c) {
        Frag<T> wf;
        wf.load(wp + 32 * c);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          Frag<T> af;
          if (aok[mt]) af.load(ap[mt] + 32 * c); else af.zero();
          acc[mt] = mma(acc[mt], af, wf);
        }
      }
    }
  }

  // accumulator tile: lane holds column ln, rows 4g..4g+3 of each 16-row tile
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][(mt * 16 + 4 * g + i) * 16 + ln] = f4get(acc[mt], i);
  __syncthreads();
  for (int i = tid; i < MP * 16; i += blockDim.x) {
    float s = 0.f;
#pragma unroll
    for (int w = 0; w < kGemmWaves; ++w) s += red[w][i];
    ct[i] = s;
  }
  __syncthreads();
  gemm_epilogue<T, EPI>(a, ct, MP, row0, t, layer);
}

template <typename T, int MT>
static hipError_t launch_mt(Epilogue epi, const GemmArgs &a, dim3 grid, hipStream_t st) {
  const dim3 block(kGemmWaves * 64);
  switch (epi) {
    case EPI_STORE: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_STORE>), grid, block, 0, st, a); break;
    case EPI_STORE_F32: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_STORE_F32>), grid, block, 0, st, a); break;
    case EPI_RESID: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_RESID>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_SWIGLU>), grid, block, 0, st, a); break;
    case EPI_QKV: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_QKV>), grid, block, 0, st, a); break;
    case EPI_INJECT: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_INJECT>), grid, block, 0, st, a); break;
    case EPI_ARGMAX: hipLaunchKernelGGL((gemm_kernel<T, MT, EPI_ARGMAX>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_gemm(bool is_bf16, Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st) {
  const int MP = gemm_rows_per_group(a.M);
  dim3 grid(a.n_groups, z_slices * a.m_groups);
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
