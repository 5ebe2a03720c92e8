// Host-side interface between the C ABI layer and the kernel launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace dflash {

constexpr int kMaxLayers = 64;

enum Epilogue {
  EPI_STORE = 0,      // out[row, col] = acc (storage type)
  EPI_STORE_F32 = 1,  // out[row, col] = acc (fp32)
  EPI_RESID = 2,      // X[row, col] += acc (fp32 residual)
  EPI_SWIGLU = 3,     // out[row, j] = silu(gate_j) * up_j (storage type)
  EPI_QKV = 4,        // RoPE(q), RoPE(k), v -> block q/k/v buffers
  EPI_INJECT = 5,     // RoPE(k), v -> paged context cache
  EPI_ARGMAX = 6,     // per-row (max, lowest argmax) over the column group
  EPI_QKV_CACHE = 7,  // EPI_QKV, and the block's k, v also into the paged cache
                      // (target verify; streaming GEMM only)
};

struct GemmArgs {
  // operands
  const void *A;          // [M, K] storage type, row stride lda
  int lda;
  const void *W[kMaxLayers];  // per z-slice weights [N_phys, K], row stride ldw
  int ldw;
  int M, N, K;            // N: output columns (SwiGLU: 2 * ffn)
  int n_groups;           // 16-column tiles (gemm_tiles)
  int m_groups;           // ceil(M / rows per group)
  // EPI_STORE / EPI_STORE_F32 / EPI_SWIGLU
  void *out;
  int ldo;
  // EPI_RESID
  float *X;
  int ldx;
  // EPI_QKV / EPI_INJECT
  void *q_out, *k_out, *v_out;
  void *kc_out, *vc_out;  // EPI_QKV_CACHE: this layer's paged cache (block k, v at ctx + j)
  const int *ctx_len;
  int block_size, nq, nkv, hd;
  double log2_theta;
  const int *seq, *pos, *block_table;
  int max_pages, page_size;
  size_t cache_layer_stride;  // elements per layer of the paged cache
  // EPI_SWIGLU
  int ffn;
  // EPI_ARGMAX
  float *amax_val;
  int *amax_idx;
  // fused activation staging (streaming GEMM): RMSNorm gain/eps, embedding gather
  const void *gain;
  float eps;
  const void *embed;
  const int *anchor;
  int mask_id;
  const int *ids;         // embedding gather: per-row token ids [M] (NULL: anchor + mask ids)
  // split-K of the LDS-tiled GEMM: fp32 partial tiles [split][M][n_groups*128]
  // (NULL: no split), bytes available there, K elements per split
  float *part;
  size_t part_bytes;
  int kper;
  // streaming GEMM's A_COPY_ROWS mode (residual projection over more than 16
  // rows): row_groups slices of the grid, one per 16-row group (grid.y); row0
  // is the group's first row, set inside the kernel
  int row_groups, row0;
  // streaming GEMM over several weight slices in one flat tile range (the
  // per-layer K/V projections of the context inject): slice = tile / n_groups;
  // 0 for one slice per grid.y index
  int z_flat;
  // streaming residual projection split over K in pairs of workgroups: one
  // arrival counter per 32-column tile (zero between launches) and the two
  // halves' fp32 partials [2][16][N]; NULL: no split
  unsigned *cnt;
  float *spart;
};

// Launch a skinny GEMM; ``z_slices`` = number of weight slices (layers) in the
// launch.  ``is_bf16`` selects the storage type.
hipError_t launch_gemm(bool is_bf16, Epilogue epi, const GemmArgs &a, int z_slices, hipStream_t st);

// Rows per GEMM workgroup for M rows (16, 32 or 64).
int gemm_rows_per_group(int M);

// Number of 16-column tiles (workgroups per row group and slice).
int gemm_tiles(Epilogue epi, int N, int ffn);

// Streaming GEMM for M <= 16 rows (persistent, one workgroup per compute unit).
// amode: 0 = activations read from global memory, 1 = copied into LDS,
// 2 = RMSNorm of the fp32 residual X into LDS, 3 = embedding gather + RMSNorm,
// 4 = copied into LDS one K-portion at a time (one tile per workgroup),
// 6 = copied into LDS, one grid slice per 16-row group (EPI_RESID only).
hipError_t launch_gemm_stream(bool is_bf16, Epilogue epi, int amode, const GemmArgs &a, int grid_x, int z_slices,
                              hipStream_t st);
// Largest K whose 16 activation rows stay resident in LDS.
int stream_res_k(bool is_bf16);

// LDS-tiled GEMM for many rows (bf16, 128 x 128 x 64 tiles).
bool gemm_tiled_ok(Epilogue epi, int N, int K, int ffn, int hd);
int gemm_tiled_cols(Epilogue epi, int N, int ffn);
hipError_t launch_gemm_tiled(Epilogue epi, GemmArgs &a, int z_slices, int cu, hipStream_t st);

struct AttnArgs {
  const void *q;          // [R, nq*hd]
  const void *kb, *vb;    // [R, nkv*hd] block keys / values
  const void *kc, *vc;    // layer base of the paged cache
  const int *block_table, *ctx_len;
  void *o;                // [R, nq*hd]
  float *partial;         // [items][GB_pad][hd] + stats
  float *stats;           // [items][GB_pad][2]
  int batch, block_size, nq, nkv, hd, max_pages, page_size, chunk, max_items;
  int causal;             // block row j sees block keys 0..j only (target verify)
  int window;             // > 0: only the last `window` context keys are attended
  const int *block_len;   // [batch] or NULL: block keys j >= block_len[s] are not attended
  int off32;              // a cache layer spans < 4 GB: byte offsets inside it fit 32 bits
};
hipError_t launch_attention(bool is_bf16, const AttnArgs &a, hipStream_t st);
int attn_chunk(int batch, int max_ctx, int block_size, int nq, int nkv, int cu);
int attn_max_items(int batch, int max_ctx, int block_size, int nkv, int chunk);

hipError_t launch_embed(bool is_bf16, const void *embed, const int *anchor, int mask_id, const int *ids, int batch,
                        int block_size, int hidden, float *X, hipStream_t st);
// Block K/V rows [batch*B, nkv*hd] of one layer into the paged cache at
// positions ctx_len[s] + j.
hipError_t launch_kv_append(bool is_bf16, const void *kb, const void *vb, void *kc, void *vc, const int *block_table,
                            const int *ctx_len, int batch, int block_size, int kvd, int max_pages, int page_size,
                            hipStream_t st);
// Residual rows X [rows, hidden] (fp32) into column block `slot` of
// taps [rows, n_slots * hidden] (storage type).
hipError_t launch_tap(bool is_bf16, const float *X, int rows, int hidden, int slot, int n_slots, void *taps,
                      hipStream_t st);
hipError_t launch_rmsnorm(bool is_bf16, const float *X, const void *gain, float eps, int rows, int hidden,
                          int block_size, bool skip_anchor, void *Y, hipStream_t st);
hipError_t launch_argmax_reduce(const float *val, const int *idx, int rows, int n_groups, int *ids_out,
                                float *max_out, hipStream_t st);
hipError_t launch_accept(const int *draft, const int *target, int batch, int block_size, const int *block_len,
                         int *tau, int *bonus, hipStream_t st);

// range check of device-resident indices (small_kernels.hip); bits as DFLASH_BAD_*
constexpr int kBadCtxLen = 1, kBadCtxPage = 2, kBadBlockPage = 4, kBadTokenId = 8, kBadInjectSlot = 16;
struct CheckArgs {
  const int *ctx_len, *block_table, *anchor, *ids, *seq, *pos;
  int batch, max_pages, n_pages, max_ctx, page_size, block_size, vocab, n_ids, n_new;
};
hipError_t launch_check_inputs(const CheckArgs &a, int *err, hipStream_t st);

// temperature sampling (sampling.hip): 1024-column chunks per workgroup
constexpr int kSampleCols = 1024;
size_t sample_ws_bytes(int rows, int vocab);
hipError_t launch_sample(const float *logits, int rows, int vocab, float inv_t, uint64_t seed, uint32_t offset,
                         uint32_t tag, int *ids_out, float *lse_out, void *ws, hipStream_t st);
hipError_t launch_accept_sample(const float *dz, const float *dlse, const int *dids, const float *tz,
                                const float *tlse, const int *tids, int batch, int B, const int *block_len,
                                int vocab, float inv_t, uint64_t seed, uint32_t offset, int *tau, int *bonus,
                                void *ws, hipStream_t st);
hipError_t launch_zero(void *p, size_t bytes, hipStream_t st);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int n_cu, hipStream_t st);

}  // namespace dflash
