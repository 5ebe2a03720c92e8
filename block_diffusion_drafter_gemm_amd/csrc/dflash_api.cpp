// C ABI of libdflash: argument validation, workspace layout and the launch
// sequence of each entry point.  All compute happens in the HIP kernels; this
// file only plans and enqueues.
#include <algorithm>
#include <cmath>
#include <math.h>
#include <string.h>

#include <mutex>
#include <new>
#include <vector>

#include "../../include/dflash.h"
#include "dflash_internal.h"

using namespace dflash;

struct dflash_handle_s {
  dflash_config cfg;
  const void *embed, *lm_head, *w_fc, *final_norm, *ctx_norm;
  const void *attn_norm[kMaxLayers], *w_qkv[kMaxLayers], *w_o[kMaxLayers];
  const void *mlp_norm[kMaxLayers], *w_gate_up[kMaxLayers], *w_down[kMaxLayers];
  bool bf16;
  size_t esz;  // bytes per stored element
  int n_cu;    // compute units of the current device (queried at the first launch)
  // measurement hook: hipEvent_t pairs around each stage of each layer (empty: off)
  std::vector<hipEvent_t> stage_events;
};

namespace {

constexpr size_t kCounterBytes = 256 * 1024;  // completion counters at the front of every workspace
constexpr size_t kAlign = 256;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

struct Carve {
  size_t off = kCounterBytes;
  size_t take(size_t bytes) {
    size_t o = off;
    off = align_up(off + bytes);
    return o;
  }
};

// ---- draft_block layout --------------------------------------------------
struct DraftLayout {
  size_t X, Y, Q, Kb, Vb, O, Hs, attn_part, attn_stats, gemm_part, gemm_part_bytes, split_part, total;
  int chunk, max_items;
};

DraftLayout draft_layout(const dflash_handle_s *h, int batch, int max_ctx, int cu) {
  const dflash_config &c = h->cfg;
  const int B = c.block_size, R = batch * B;
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  DraftLayout L;
  Carve cv;
  L.X = cv.take((size_t)R * c.hidden * 4);
  L.Y = cv.take((size_t)R * c.hidden * h->esz);
  L.Q = cv.take((size_t)R * qd * h->esz);
  L.Kb = cv.take((size_t)R * kvd * h->esz);
  L.Vb = cv.take((size_t)R * kvd * h->esz);
  L.O = cv.take((size_t)R * qd * h->esz);
  L.Hs = cv.take((size_t)R * c.ffn * h->esz);
  // a sliding window bounds the attended context (and so the chunk items)
  const int att_ctx = c.window > 0 && c.window < max_ctx ? c.window : max_ctx;
  L.chunk = attn_chunk(batch, att_ctx, B, c.n_q_heads, c.n_kv_heads, cu);
  L.max_items = attn_max_items(batch, att_ctx, B, c.n_kv_heads, L.chunk);
  const int GB = (c.n_q_heads / c.n_kv_heads) * B, GBP = (GB + 15) / 16 * 16;
  L.attn_part = cv.take((size_t)L.max_items * GBP * c.head_dim * 4);
  L.attn_stats = cv.take((size_t)L.max_items * GBP * 2 * 4);
  // split-K partials of the residual projections (O, down) of the many-rows
  // path: up to 4 fp32 slices of [R, hidden]
  L.gemm_part_bytes = R > 64 ? (size_t)4 * R * c.hidden * 4 : 0;
  L.gemm_part = cv.take(L.gemm_part_bytes);
  // the two halves' partials of the split residual projection (<= 16 rows);
  // reserved whenever one sequence's block fits, so that a smaller batch never
  // needs more workspace than the largest
  L.split_part = B <= 16 ? cv.take((size_t)2 * 16 * c.hidden * 4) : 0;
  L.total = cv.off;
  return L;
}

struct LmLayout {
  size_t val, idx, total;
};

LmLayout lm_layout(const dflash_handle_s *h, int rows) {
  const dflash_config &c = h->cfg;
  LmLayout L;
  Carve cv;
  const int ng = gemm_tiles(EPI_ARGMAX, c.vocab, c.ffn);
  L.val = cv.take((size_t)rows * ng * 4);
  L.idx = cv.take((size_t)rows * ng * 4);
  L.total = cv.off;
  return L;
}

struct InjectLayout {
  size_t c, cf, total;
};

InjectLayout inject_layout(const dflash_handle_s *h, int n_new) {
  const dflash_config &c = h->cfg;
  InjectLayout L;
  Carve cv;
  L.c = cv.take((size_t)n_new * c.hidden * h->esz);
  L.cf = c.ctx_norm ? cv.take((size_t)n_new * c.hidden * 4) : 0;   // fp32 projection before the norm
  L.total = cv.off;
  return L;
}

int compute_units(dflash_handle_s *h);

// Kernel choice of launch(): the LDS-tiled kernel for many rows (bf16), and for
// 17..64 rows when its 128-row tiles still number at least 64 (wide outputs: LM
// head, gate/up); otherwise the few-rows kernel.
bool use_tiled(const dflash_handle_s *h, Epilogue epi, int M, int N, int K, int ffn, int hd, int z) {
  const bool tiled_ok = h->bf16 && gemm_tiled_ok(epi, N, K, ffn, hd);
  return tiled_ok && (M > 64 || (M > 16 && gemm_tiled_cols(epi, N, ffn) * z >= 64));
}

// Whether launch() can take this GEMM: the few-rows kernel puts its row groups
// times the weight slices in grid.y (at most 65535).  Checked for every GEMM of
// a call before that call enqueues anything.
int gemm_fits(const dflash_handle_s *h, Epilogue epi, int M, int N, int K, int ffn, int hd, int z) {
  if (use_tiled(h, epi, M, N, K, ffn, hd, z)) return DFLASH_OK;
  const int MP = gemm_rows_per_group(M);
  return (long)((M + MP - 1) / MP) * z > 65535 ? DFLASH_ERR_SHAPE : DFLASH_OK;
}

// Fill the launch geometry of ``a`` and launch (the kernel choice of use_tiled;
// the caller has checked gemm_fits).
int launch(const dflash_handle_s *h, Epilogue epi, GemmArgs &a, int z, hipStream_t st) {
  if (use_tiled(h, epi, a.M, a.N, a.K, a.ffn, a.hd, z)) {
    a.m_groups = 1;
    a.n_groups = gemm_tiled_cols(epi, a.N, a.ffn);
    return launch_gemm_tiled(epi, a, z, compute_units(const_cast<dflash_handle_s *>(h)), st) == hipSuccess
               ? DFLASH_OK
               : DFLASH_ERR_HIP;
  }
  const int MP = gemm_rows_per_group(a.M);
  a.m_groups = (a.M + MP - 1) / MP;
  a.n_groups = gemm_tiles(epi, a.N, a.ffn);
  if ((long)a.m_groups * z > 65535) return DFLASH_ERR_SHAPE;   // unreachable after gemm_fits
  return launch_gemm(h->bf16, epi, a, z, st) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int compute_units(dflash_handle_s *h) {
  if (h->n_cu <= 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    h->n_cu = n;
  }
  return h->n_cu;
}

enum {
  AM_GLOBAL = 0, AM_COPY = 1, AM_NORM = 2, AM_EMBED_NORM = 3, AM_PORTION = 4, AM_COPY_ROWS = 6, AM_TW8 = 16,
  AM_SPLIT2 = 32
};

// Streaming GEMM (M <= 16): one persistent workgroup per compute unit.
int launch_stream(dflash_handle_s *h, Epilogue epi, int amode, GemmArgs &a, int z, hipStream_t st,
                  int *grid_out = nullptr) {
  a.m_groups = 1;
  a.n_groups = gemm_tiles(epi, a.N, a.ffn);
  const int cu = compute_units(h);
  // bf16 QKV with RMSNorm staging: 8-column tiles (4 RoPE pairs) where they
  // lower the weight bytes of the busiest workgroup (384 16-column tiles on
  // 256 compute units: 2 per workgroup on 192 of them; 768 8-column tiles: 3
  // per workgroup on all 256)
  if (h->bf16 && (epi == EPI_QKV || epi == EPI_QKV_CACHE) && (amode == AM_NORM || amode == AM_EMBED_NORM) &&
      a.hd % 8 == 0 && a.K % 64 == 0) {
    const int per16 = (a.n_groups + cu - 1) / cu, per8 = (2 * a.n_groups + cu - 1) / cu;
    if (per8 < 2 * per16) {
      amode |= AM_TW8;
      a.n_groups *= 2;
    }
  }
  // bf16 residual projection with K past the resident capacity (the down
  // projection): 32-column tiles in pairs of workgroups, each over half of K,
  // so a compute unit reads half the activation bytes for the same weight
  // bytes; the pair's second workgroup to finish adds both halves
  if (h->bf16 && epi == EPI_RESID && amode == AM_GLOBAL && z == 1 && a.cnt && a.spart &&
      a.K > stream_res_k(true) && a.K % 128 == 0 && a.N % 256 == 0 && a.N / 16 <= cu) {
    a.z_flat = 0;
    const int grid = a.N / 16;   // 2 x the 32-column tiles
    a.n_groups = grid;
    if (grid_out) *grid_out = grid;
    return launch_gemm_stream(true, epi, AM_SPLIT2, a, grid, 1, st) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
  }
  // several weight slices (the inject's per-layer K/V projections): one flat
  // tile range over all of them, so a workgroup stages its rows once for tiles
  // of several slices (5 layers x 128 tiles on 256 compute units: 3 tiles per
  // workgroup in one launch round instead of 640 one-tile workgroups)
  a.z_flat = 0;
  if (z > 1 && epi == EPI_INJECT && (amode == AM_COPY || amode == AM_GLOBAL)) {
    a.z_flat = z;
    z = 1;
  }
  const int tiles = a.n_groups * (a.z_flat > 0 ? a.z_flat : 1);
  // the fewest workgroups that keep the largest per-workgroup tile count (a
  // balanced grid); portions run one tile per workgroup
  const int per = (tiles + cu - 1) / cu;
  int grid = (tiles + per - 1) / per;
  if (amode == AM_PORTION) grid = a.n_groups;
  if (grid_out) *grid_out = grid;
  return launch_gemm_stream(h->bf16, epi, amode, a, grid, z, st) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

// Residual projection or LM head argmax (K within the LDS capacity) over
// 17..64 rows on the streaming GEMM: one grid slice per 16-row group (grid.y).
// Each slice gets an equal share of the compute units, a multiple of 8, so
// that the slices' workgroups for one column tile run on the same XCD and its
// L2 serves them the weights after the first read.
int launch_rows(dflash_handle_s *h, Epilogue epi, GemmArgs &a, hipStream_t st, int *grid_out = nullptr) {
  const int groups = (a.M + 15) / 16;
  a.row_groups = groups;
  a.z_flat = 0;
  a.m_groups = 1;
  a.n_groups = gemm_tiles(epi, a.N, a.ffn);
  int cu = compute_units(h) / groups / 8 * 8;
  if (cu < 8) cu = 8;
  const int per = (a.n_groups + cu - 1) / cu;
  int grid = (a.n_groups + per - 1) / per;        // <= n_groups: every workgroup has a tile
  // a multiple of 8 keeps a tile's workgroups of all slices on one XCD; only
  // where that still gives every workgroup a tile
  const int g8 = (grid + 7) / 8 * 8;
  if (g8 <= cu && g8 <= a.n_groups) grid = g8;
  if (grid_out) *grid_out = grid;
  return launch_gemm_stream(h->bf16, epi, AM_COPY_ROWS, a, grid, groups, st) == hipSuccess ? DFLASH_OK
                                                                                         : DFLASH_ERR_HIP;
}

int validate_config(const dflash_config *c) {
  if (c->dtype != DFLASH_F32 && c->dtype != DFLASH_BF16) return DFLASH_ERR_DTYPE;
  if (c->hidden <= 0 || c->hidden % 64 || c->hidden > 16384) return DFLASH_ERR_SHAPE;
  if (c->head_dim != 64 && c->head_dim != 128) return DFLASH_ERR_SHAPE;
  if (c->n_q_heads <= 0 || c->n_kv_heads <= 0 || c->n_q_heads % c->n_kv_heads) return DFLASH_ERR_SHAPE;
  if ((c->n_q_heads * c->head_dim) % 64) return DFLASH_ERR_SHAPE;
  if (c->ffn <= 0 || c->ffn % 64) return DFLASH_ERR_SHAPE;
  if (c->vocab <= 0 || c->vocab % 16) return DFLASH_ERR_SHAPE;
  if (c->n_layers < 1 || c->n_layers > kMaxLayers) return DFLASH_ERR_SHAPE;
  if (c->n_feat_layers < 1) return DFLASH_ERR_SHAPE;
  if (c->block_size < 2 || c->block_size > 64) return DFLASH_ERR_SHAPE;
  if ((c->n_q_heads / c->n_kv_heads) * c->block_size > 128) return DFLASH_ERR_SHAPE;
  if (c->page_size != 16) return DFLASH_ERR_SHAPE;
  if (c->mask_token_id < 0 || c->mask_token_id >= c->vocab) return DFLASH_ERR_RANGE;
  if (!(c->rope_theta > 0.f) || !(c->rms_eps >= 0.f)) return DFLASH_ERR_RANGE;
  if (c->window < 0) return DFLASH_ERR_RANGE;
  if (c->ctx_norm != 0 && c->ctx_norm != 1) return DFLASH_ERR_RANGE;
  return DFLASH_OK;
}

int validate_kv(const dflash_handle_s *h, const dflash_kv *kv) {
  if (!kv) return DFLASH_ERR_NULL;
  if (!kv->k || !kv->v || !kv->block_table || !kv->ctx_len) return DFLASH_ERR_NULL;
  // cache rows are read and written in 16-byte pieces
  if (reinterpret_cast<uintptr_t>(kv->k) % 16 || reinterpret_cast<uintptr_t>(kv->v) % 16) return DFLASH_ERR_RANGE;
  if (kv->batch < 1 || kv->max_pages < 1 || kv->n_pages < 1 || kv->max_ctx < 0) return DFLASH_ERR_SHAPE;
  (void)h;
  return DFLASH_OK;
}

}  // namespace

// Scratch memory of dflash_lmhead_argmax_noalloc: the argmax partials live in
// this array instead of a caller workspace.  Each device holds its own copy,
// at its own address, until the process ends.  Host code never passes the
// array's name to a kernel (on the host it is only a stand-in for the symbol):
// it passes the device address hipGetSymbolAddress returns, looked up once per
// device with that device current.
constexpr size_t kScratchBytes = size_t(8) << 20;
constexpr int kMaxDevices = 64;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];
static std::mutex g_scratch_mu;
static void *g_scratch_addr[kMaxDevices];

static int scratch_on_current_device(void **out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) return DFLASH_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return DFLASH_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_addr[dev]) {
    void *p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return DFLASH_ERR_HIP;
    g_scratch_addr[dev] = p;
  }
  *out = g_scratch_addr[dev];
  return DFLASH_OK;
}

extern "C" {

const char *dflash_status_str(int status) {
  switch (status) {
    case DFLASH_OK: return "ok";
    case DFLASH_ERR_NULL: return "null pointer argument";
    case DFLASH_ERR_SHAPE: return "unsupported or inconsistent shape";
    case DFLASH_ERR_DTYPE: return "unknown storage type";
    case DFLASH_ERR_RANGE: return "value out of range";
    case DFLASH_ERR_WORKSPACE: return "workspace too small";
    case DFLASH_ERR_UNSUPPORTED: return "unsupported combination";
    case DFLASH_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int dflash_create(const dflash_config *cfg, const dflash_weights *w, dflash_handle *out) {
  if (!cfg || !w || !out) return DFLASH_ERR_NULL;
  *out = nullptr;
  int st = validate_config(cfg);
  if (st != DFLASH_OK) return st;
  if (!w->embed || !w->lm_head || !w->final_norm || !w->attn_norm || !w->w_qkv || !w->w_o ||
      !w->mlp_norm || !w->w_gate_up || !w->w_down)
    return DFLASH_ERR_NULL;
  for (int l = 0; l < cfg->n_layers; ++l)
    if (!w->attn_norm[l] || !w->w_qkv[l] || !w->w_o[l] || !w->mlp_norm[l] || !w->w_gate_up[l] || !w->w_down[l])
      return DFLASH_ERR_NULL;
  if (cfg->ctx_norm && !w->ctx_norm) return DFLASH_ERR_NULL;
  dflash_handle_s *h = new (std::nothrow) dflash_handle_s();
  if (!h) return DFLASH_ERR_RANGE;
  h->cfg = *cfg;
  h->embed = w->embed;
  h->lm_head = w->lm_head;
  h->w_fc = w->w_fc;
  h->final_norm = w->final_norm;
  h->ctx_norm = cfg->ctx_norm ? w->ctx_norm : nullptr;
  for (int l = 0; l < cfg->n_layers; ++l) {
    h->attn_norm[l] = w->attn_norm[l];
    h->w_qkv[l] = w->w_qkv[l];
    h->w_o[l] = w->w_o[l];
    h->mlp_norm[l] = w->mlp_norm[l];
    h->w_gate_up[l] = w->w_gate_up[l];
    h->w_down[l] = w->w_down[l];
  }
  h->bf16 = cfg->dtype == DFLASH_BF16;
  h->esz = h->bf16 ? 2 : 4;
  *out = h;
  return DFLASH_OK;
}

int dflash_destroy(dflash_handle h) {
  if (!h) return DFLASH_ERR_NULL;
  delete h;
  return DFLASH_OK;
}

int dflash_workspace_size(dflash_handle h, int32_t max_batch, int32_t max_ctx, int32_t max_new, size_t *bytes) {
  if (!h || !bytes) return DFLASH_ERR_NULL;
  if (max_batch < 1 || max_ctx < 0 || max_new < 0) return DFLASH_ERR_SHAPE;
  size_t need = draft_layout(h, max_batch, max_ctx, compute_units(h)).total;
  const size_t lm = lm_layout(h, max_batch * (h->cfg.block_size - 1)).total;
  const size_t inj = inject_layout(h, max_new).total;
  need = need > lm ? need : lm;
  need = need > inj ? need : inj;
  *bytes = need;
  return DFLASH_OK;
}

int dflash_workspace_init(dflash_handle h, void *ws, size_t ws_bytes, void *stream) {
  if (!h || !ws) return DFLASH_ERR_NULL;
  if (ws_bytes < kCounterBytes) return DFLASH_ERR_WORKSPACE;
  return launch_zero(ws, kCounterBytes, (hipStream_t)stream) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int dflash_inject_context(dflash_handle h, const void *feats, const int32_t *seq, const int32_t *pos, int32_t n_new,
                          const dflash_kv *kv, void *ws, size_t ws_bytes, void *stream) {
  if (!h) return DFLASH_ERR_NULL;
  if (n_new < 0) return DFLASH_ERR_SHAPE;
  int st = validate_kv(h, kv);
  if (st != DFLASH_OK) return st;
  if (n_new == 0) return DFLASH_OK;
  if (!feats || !seq || !pos || !ws || !h->w_fc) return DFLASH_ERR_NULL;
  const dflash_config &c = h->cfg;
  const InjectLayout L = inject_layout(h, n_new);
  if (ws_bytes < L.total) return DFLASH_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  hipStream_t s = (hipStream_t)stream;
  const int kvd = c.n_kv_heads * c.head_dim, qd = c.n_q_heads * c.head_dim;
  const int KR = stream_res_k(h->bf16);
  const bool small = n_new <= 16;
  // every launch shape is checked before anything is enqueued
  if (!small && (gemm_fits(h, c.ctx_norm ? EPI_STORE_F32 : EPI_STORE, n_new, c.hidden, c.n_feat_layers * c.hidden,
                           0, 0, 1) != DFLASH_OK ||
                 gemm_fits(h, EPI_INJECT, n_new, 2 * kvd, c.hidden, 0, c.head_dim, c.n_layers) != DFLASH_OK))
    return DFLASH_ERR_SHAPE;

  // A1: c = feats * W_fc^T (then RMSNorm(c) when the handle has ctx_norm)
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = feats;
  a.lda = c.n_feat_layers * c.hidden;
  a.W[0] = h->w_fc;
  a.ldw = c.n_feat_layers * c.hidden;
  a.M = n_new;
  a.N = c.hidden;
  a.K = c.n_feat_layers * c.hidden;
  a.out = w + (c.ctx_norm ? L.cf : L.c);
  a.ldo = c.hidden;
  const Epilogue fe = c.ctx_norm ? EPI_STORE_F32 : EPI_STORE;
  st = small ? launch_stream(h, fe, a.K <= KR ? AM_COPY : AM_PORTION, a, 1, s) : launch(h, fe, a, 1, s);
  if (st != DFLASH_OK) return st;
  if (c.ctx_norm && launch_rmsnorm(h->bf16, reinterpret_cast<const float *>(w + L.cf), h->ctx_norm, c.rms_eps,
                                   n_new, c.hidden, 1, false, w + L.c, s) != hipSuccess)
    return DFLASH_ERR_HIP;

  // A2: every layer's K and V projections of c, RoPE on K, paged write
  GemmArgs b;
  memset(&b, 0, sizeof(b));
  b.A = w + L.c;
  b.lda = c.hidden;
  for (int l = 0; l < c.n_layers; ++l)
    b.W[l] = static_cast<const char *>(h->w_qkv[l]) + (size_t)qd * c.hidden * h->esz;
  b.ldw = c.hidden;
  b.M = n_new;
  b.N = 2 * kvd;
  b.K = c.hidden;
  b.k_out = kv->k;
  b.v_out = kv->v;
  b.nq = c.n_q_heads;
  b.nkv = c.n_kv_heads;
  b.hd = c.head_dim;
  b.log2_theta = log2((double)c.rope_theta);
  b.seq = seq;
  b.pos = pos;
  b.block_table = kv->block_table;
  b.max_pages = kv->max_pages;
  b.page_size = c.page_size;
  b.cache_layer_stride = (size_t)kv->n_pages * c.page_size * kvd;
  return small ? launch_stream(h, EPI_INJECT, c.hidden <= KR ? AM_COPY : AM_GLOBAL, b, c.n_layers, s)
               : launch(h, EPI_INJECT, b, c.n_layers, s);
}

// Records the measurement hook's event for (layer, stage), before (end = 0) or
// after (end = 1) the stage's launches; nothing when the hook is off.
static int mark_stage(const dflash_handle_s *h, int layer, int stage, int end, hipStream_t s) {
  if (h->stage_events.empty()) return DFLASH_OK;
  const size_t i = 2 * ((size_t)layer * DFLASH_N_STAGES + stage) + end;
  return hipEventRecord(h->stage_events[i], s) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

// One pass of the handle's decoder over a block of B rows per sequence at
// positions ctx_len[s] .. ctx_len[s] + B - 1.  Drafter (ids == NULL): rows are
// the anchor and B - 1 mask tokens, attention is non-causal, the context cache
// is only read and the final norm covers the mask rows.  Target verify (ids
// set): rows are the given tokens, attention is causal within the block, every
// layer's block K/V are appended to the cache, the residual rows after the
// tapped layers go to taps_out and the final norm covers all B rows.
static int forward_block(dflash_handle h, const int32_t *anchor_ids, const int32_t *ids, const int32_t *tap_layers,
                         int32_t n_taps, void *taps_out, const dflash_kv *kv, void *hidden_out, void *ws,
                         size_t ws_bytes, hipStream_t s) {
  int st = DFLASH_OK;
  const bool verify = ids != nullptr;
  const dflash_config &c = h->cfg;
  const int B = c.block_size, batch = kv->batch, R = batch * B;
  const DraftLayout L = draft_layout(h, batch, kv->max_ctx, compute_units(h));
  if (ws_bytes < L.total) return DFLASH_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  const int qd = c.n_q_heads * c.head_dim, kvd = c.n_kv_heads * c.head_dim;
  float *X = reinterpret_cast<float *>(w + L.X);
  const size_t cache_layer = (size_t)kv->n_pages * c.page_size * kvd * h->esz;
  const int KR = stream_res_k(h->bf16);
  // streaming path: up to 16 block rows, hidden states resident in LDS (norms fused)
  const bool fast = R <= 16 && c.hidden <= KR && qd <= KR;
  // 17..64 rows: the O projection on the streaming GEMM once per 16-row group
  // (measured against the few-rows GEMM at 64 rows: O 26.4 -> 15.4 us; QKV and
  // down were slower that way and keep their kernels)
  const bool sliced = !fast && R <= 64 && qd <= KR;
  // every launch shape is checked before anything is enqueued
  if (!fast && (gemm_fits(h, EPI_QKV, R, qd + 2 * kvd, c.hidden, 0, c.head_dim, 1) != DFLASH_OK ||
                (!sliced && gemm_fits(h, EPI_RESID, R, c.hidden, qd, 0, 0, 1) != DFLASH_OK) ||
                gemm_fits(h, EPI_SWIGLU, R, 2 * c.ffn, c.hidden, c.ffn, 0, 1) != DFLASH_OK ||
                gemm_fits(h, EPI_RESID, R, c.hidden, c.ffn, 0, 0, 1) != DFLASH_OK))
    return DFLASH_ERR_SHAPE;

  if (!fast &&
      launch_embed(h->bf16, h->embed, anchor_ids, c.mask_token_id, ids, batch, B, c.hidden, X, s) != hipSuccess)
    return DFLASH_ERR_HIP;
  for (int l = 0; l < c.n_layers; ++l) {
    // A4: RMSNorm, QKV projection, RoPE; block q/k/v to the workspace
    if ((st = mark_stage(h, l, DFLASH_STAGE_QKV, 0, s)) != DFLASH_OK) return st;
    GemmArgs q;
    memset(&q, 0, sizeof(q));
    q.W[0] = h->w_qkv[l];
    q.ldw = c.hidden;
    q.M = R;
    q.N = qd + 2 * kvd;
    q.K = c.hidden;
    q.q_out = w + L.Q;
    q.k_out = w + L.Kb;
    q.v_out = w + L.Vb;
    q.ctx_len = kv->ctx_len;
    q.block_size = B;
    q.nq = c.n_q_heads;
    q.nkv = c.n_kv_heads;
    q.hd = c.head_dim;
    q.log2_theta = log2((double)c.rope_theta);
    if (fast) {
      q.X = X;
      q.ldx = c.hidden;
      q.gain = h->attn_norm[l];
      q.eps = c.rms_eps;
      q.embed = h->embed;
      q.anchor = anchor_ids;
      q.mask_id = c.mask_token_id;
      q.ids = ids;
      if (verify) {   // the block's k, v go to the cache from the QKV epilogue
        q.kc_out = static_cast<char *>(kv->k) + l * cache_layer;
        q.vc_out = static_cast<char *>(kv->v) + l * cache_layer;
        q.block_table = kv->block_table;
        q.max_pages = kv->max_pages;
        q.page_size = c.page_size;
      }
      st = launch_stream(h, verify ? EPI_QKV_CACHE : EPI_QKV, l == 0 ? AM_EMBED_NORM : AM_NORM, q, 1, s);
    } else {
      if (launch_rmsnorm(h->bf16, X, h->attn_norm[l], c.rms_eps, R, c.hidden, B, false, w + L.Y, s) != hipSuccess)
        return DFLASH_ERR_HIP;
      q.A = w + L.Y;
      q.lda = c.hidden;
      st = launch(h, EPI_QKV, q, 1, s);
    }
    if (st != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_QKV, 1, s)) != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_ATTENTION, 0, s)) != DFLASH_OK) return st;

    // A5: attention over the paged context plus the block, no mask
    AttnArgs at;
    memset(&at, 0, sizeof(at));
    at.q = w + L.Q;
    at.kb = w + L.Kb;
    at.vb = w + L.Vb;
    at.kc = static_cast<const char *>(kv->k) + l * cache_layer;
    at.vc = static_cast<const char *>(kv->v) + l * cache_layer;
    at.block_table = kv->block_table;
    at.ctx_len = kv->ctx_len;
    at.o = w + L.O;
    at.partial = reinterpret_cast<float *>(w + L.attn_part);
    at.stats = reinterpret_cast<float *>(w + L.attn_stats);
    at.batch = batch;
    at.block_size = B;
    at.nq = c.n_q_heads;
    at.nkv = c.n_kv_heads;
    at.hd = c.head_dim;
    at.max_pages = kv->max_pages;
    at.page_size = c.page_size;
    at.chunk = L.chunk;
    at.max_items = L.max_items;
    at.causal = verify ? 1 : 0;
    at.window = c.window;
    at.block_len = kv->block_len;
    at.off32 = (uint64_t)cache_layer < (1ull << 32) ? 1 : 0;
    if (launch_attention(h->bf16, at, s) != hipSuccess) return DFLASH_ERR_HIP;
    // target verify: the block's K/V join the context cache (the caller keeps
    // the accepted positions by advancing ctx_len; later blocks overwrite the rest)
    // (the streaming path's QKV epilogue has already written them)
    if (verify && !fast &&
        launch_kv_append(h->bf16, w + L.Kb, w + L.Vb, static_cast<char *>(kv->k) + l * cache_layer,
                                   static_cast<char *>(kv->v) + l * cache_layer, kv->block_table, kv->ctx_len, batch,
                                   B, kvd, kv->max_pages, c.page_size, s) != hipSuccess)
      return DFLASH_ERR_HIP;
    if ((st = mark_stage(h, l, DFLASH_STAGE_ATTENTION, 1, s)) != DFLASH_OK) return st;

    // A6: O projection + residual
    if ((st = mark_stage(h, l, DFLASH_STAGE_O, 0, s)) != DFLASH_OK) return st;
    GemmArgs o;
    memset(&o, 0, sizeof(o));
    o.A = w + L.O;
    o.lda = qd;
    o.W[0] = h->w_o[l];
    o.ldw = qd;
    o.M = R;
    o.N = c.hidden;
    o.K = qd;
    o.X = X;
    o.ldx = c.hidden;
    o.part = L.gemm_part_bytes ? reinterpret_cast<float *>(w + L.gemm_part) : nullptr;
    o.part_bytes = L.gemm_part_bytes;
    // one tile per workgroup: activation fragments read straight from L2 beat
    // staging the rows through LDS first
    st = fast     ? launch_stream(h, EPI_RESID, AM_GLOBAL, o, 1, s)
         : sliced ? launch_rows(h, EPI_RESID, o, s)
                  : launch(h, EPI_RESID, o, 1, s);
    if (st != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_O, 1, s)) != DFLASH_OK) return st;

    // A7: RMSNorm, gate/up + SwiGLU, down + residual
    if ((st = mark_stage(h, l, DFLASH_STAGE_GATE_UP, 0, s)) != DFLASH_OK) return st;
    GemmArgs gu;
    memset(&gu, 0, sizeof(gu));
    gu.W[0] = h->w_gate_up[l];
    gu.ldw = c.hidden;
    gu.M = R;
    gu.N = 2 * c.ffn;
    gu.K = c.hidden;
    gu.ffn = c.ffn;
    gu.out = w + L.Hs;
    gu.ldo = c.ffn;
    if (fast) {
      gu.X = X;
      gu.ldx = c.hidden;
      gu.gain = h->mlp_norm[l];
      gu.eps = c.rms_eps;
      st = launch_stream(h, EPI_SWIGLU, AM_NORM, gu, 1, s);
    } else {
      if (launch_rmsnorm(h->bf16, X, h->mlp_norm[l], c.rms_eps, R, c.hidden, B, false, w + L.Y, s) != hipSuccess)
        return DFLASH_ERR_HIP;
      gu.A = w + L.Y;
      gu.lda = c.hidden;
      st = launch(h, EPI_SWIGLU, gu, 1, s);
    }
    if (st != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_GATE_UP, 1, s)) != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_DOWN, 0, s)) != DFLASH_OK) return st;

    GemmArgs dn;
    memset(&dn, 0, sizeof(dn));
    dn.A = w + L.Hs;
    dn.lda = c.ffn;
    dn.W[0] = h->w_down[l];
    dn.ldw = c.ffn;
    dn.M = R;
    dn.N = c.hidden;
    dn.K = c.ffn;
    dn.X = X;
    dn.ldx = c.hidden;
    dn.part = o.part;
    dn.part_bytes = o.part_bytes;
    if (L.split_part && R <= 16) {   // arrival counters at the front of the workspace
      dn.cnt = reinterpret_cast<unsigned *>(w);
      dn.spart = reinterpret_cast<float *>(w + L.split_part);
    }
    st = fast ? launch_stream(h, EPI_RESID, c.ffn <= KR ? AM_COPY : AM_GLOBAL, dn, 1, s)
              : launch(h, EPI_RESID, dn, 1, s);
    if (st != DFLASH_OK) return st;
    if ((st = mark_stage(h, l, DFLASH_STAGE_DOWN, 1, s)) != DFLASH_OK) return st;
    for (int i = 0; i < n_taps; ++i)   // target hidden-state taps after this layer
      if (tap_layers[i] == l && launch_tap(h->bf16, X, R, c.hidden, i, n_taps, taps_out, s) != hipSuccess)
        return DFLASH_ERR_HIP;
  }
  // A8: final RMSNorm (drafter: the mask rows; target: every row)
  const int out_rows = verify ? R : batch * (B - 1);
  if (launch_rmsnorm(h->bf16, X, h->final_norm, c.rms_eps, out_rows, c.hidden, B, !verify, hidden_out, s) !=
      hipSuccess)
    return DFLASH_ERR_HIP;
  return DFLASH_OK;
}

int dflash_set_stage_events(dflash_handle h, void *const *events, int32_t n_events) {
  if (!h) return DFLASH_ERR_NULL;
  if (!events) {
    h->stage_events.clear();
    return DFLASH_OK;
  }
  if (n_events != 2 * DFLASH_N_STAGES * h->cfg.n_layers) return DFLASH_ERR_SHAPE;
  for (int i = 0; i < n_events; ++i)
    if (!events[i]) return DFLASH_ERR_NULL;
  h->stage_events.assign(reinterpret_cast<const hipEvent_t *>(events),
                         reinterpret_cast<const hipEvent_t *>(events) + n_events);
  return DFLASH_OK;
}

int dflash_draft_block(dflash_handle h, const int32_t *anchor_ids, const dflash_kv *kv, void *hidden_out, void *ws,
                       size_t ws_bytes, void *stream) {
  if (!h) return DFLASH_ERR_NULL;
  int st = validate_kv(h, kv);
  if (st != DFLASH_OK) return st;
  if (!anchor_ids || !hidden_out || !ws) return DFLASH_ERR_NULL;
  return forward_block(h, anchor_ids, nullptr, nullptr, 0, nullptr, kv, hidden_out, ws, ws_bytes,
                       (hipStream_t)stream);
}

int dflash_target_verify(dflash_handle h, const int32_t *ids, const dflash_kv *kv, const int32_t *tap_layers,
                         int32_t n_taps, void *taps_out, void *hidden_out, void *ws, size_t ws_bytes, void *stream) {
  if (!h) return DFLASH_ERR_NULL;
  int st = validate_kv(h, kv);
  if (st != DFLASH_OK) return st;
  if (!ids || !hidden_out || !ws) return DFLASH_ERR_NULL;
  if (n_taps < 0 || n_taps > kMaxLayers) return DFLASH_ERR_SHAPE;
  if (n_taps > 0 && (!tap_layers || !taps_out)) return DFLASH_ERR_NULL;
  for (int i = 0; i < n_taps; ++i)
    if (tap_layers[i] < 0 || tap_layers[i] >= h->cfg.n_layers) return DFLASH_ERR_RANGE;
  return forward_block(h, nullptr, ids, tap_layers, n_taps, taps_out, kv, hidden_out, ws, ws_bytes,
                       (hipStream_t)stream);
}

}  // extern "C"

// The LM head and its argmax over ``rows`` hidden rows with the argmax partials
// in ``ws`` (the caller's workspace, or the scratch array); arguments checked
// by the entry points.
static int lmhead_argmax_impl(dflash_handle h, const void *hidden, int32_t rows, int32_t *ids_out,
                              float *max_logit_out, float *logits_out, void *ws, size_t ws_bytes, void *stream) {
  const dflash_config &c = h->cfg;
  const LmLayout L = lm_layout(h, rows);
  if (ws_bytes < L.total) return DFLASH_ERR_WORKSPACE;
  char *w = static_cast<char *>(ws);
  hipStream_t s = (hipStream_t)stream;
  const bool small = rows <= 16;
  const int KR = stream_res_k(h->bf16);
  // 17..32 rows with resident K: two 16-row groups sharing each weight tile
  // through L2 (with more groups each slice's compute units stream too many
  // tiles: 60 rows took 524 us against 181 us on the LDS-tiled path)
  const bool grouped = !small && rows <= 32 && c.hidden <= KR;
  if (!small && !grouped &&
      (gemm_fits(h, EPI_ARGMAX, rows, c.vocab, c.hidden, 0, 0, 1) != DFLASH_OK ||
       gemm_fits(h, EPI_STORE_F32, rows, c.vocab, c.hidden, 0, 0, 1) != DFLASH_OK))
    return DFLASH_ERR_SHAPE;
  GemmArgs a;
  memset(&a, 0, sizeof(a));
  a.A = hidden;
  a.lda = c.hidden;
  a.W[0] = h->lm_head;
  a.ldw = c.hidden;
  a.M = rows;
  a.N = c.vocab;
  a.K = c.hidden;
  a.amax_val = reinterpret_cast<float *>(w + L.val);
  a.amax_idx = reinterpret_cast<int *>(w + L.idx);
  const int am = c.hidden <= KR ? AM_COPY : AM_GLOBAL;
  int parts = 0;
  int st = DFLASH_OK;
  if (!ids_out) {   // logits only
    a.out = logits_out;
    a.ldo = c.vocab;
    return small ? launch_stream(h, EPI_STORE_F32, am, a, 1, s) : launch(h, EPI_STORE_F32, a, 1, s);
  }
  st = small     ? launch_stream(h, EPI_ARGMAX, am, a, 1, s, &parts)
       : grouped ? launch_rows(h, EPI_ARGMAX, a, s, &parts)
                 : launch(h, EPI_ARGMAX, a, 1, s);
  if (st != DFLASH_OK) return st;
  if (!small && !grouped) parts = a.n_groups;
  if (launch_argmax_reduce(a.amax_val, a.amax_idx, rows, parts, ids_out, max_logit_out, s) != hipSuccess)
    return DFLASH_ERR_HIP;
  if (logits_out) {
    GemmArgs b = a;
    b.out = logits_out;
    b.ldo = c.vocab;
    st = small ? launch_stream(h, EPI_STORE_F32, am, b, 1, s) : launch(h, EPI_STORE_F32, b, 1, s);
    if (st != DFLASH_OK) return st;
  }
  return DFLASH_OK;
}

extern "C" {

int dflash_lmhead_argmax(dflash_handle h, const void *hidden, int32_t rows, int32_t *ids_out, float *max_logit_out,
                         float *logits_out, void *ws, size_t ws_bytes, void *stream) {
  if (!h) return DFLASH_ERR_NULL;
  if (rows < 0) return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!hidden || !ws || (!ids_out && !logits_out)) return DFLASH_ERR_NULL;
  return lmhead_argmax_impl(h, hidden, rows, ids_out, max_logit_out, logits_out, ws, ws_bytes, stream);
}

int dflash_lmhead_argmax_noalloc(dflash_handle h, const void *hidden, int32_t rows, int32_t *ids_out,
                                 float *max_logit_out, void *stream) {
  if (!h) return DFLASH_ERR_NULL;
  if (rows < 0) return DFLASH_ERR_SHAPE;
  if (rows == 0) return DFLASH_OK;
  if (!hidden || !ids_out) return DFLASH_ERR_NULL;
  if (lm_layout(h, rows).total > kScratchBytes) return DFLASH_ERR_WORKSPACE;
  void *scr = nullptr;
  const int st = scratch_on_current_device(&scr);
  if (st != DFLASH_OK) return st;
  return lmhead_argmax_impl(h, hidden, rows, ids_out, max_logit_out, nullptr, scr, kScratchBytes, stream);
}

int dflash_accept_len(const int32_t *draft_ids, const int32_t *target_ids, int32_t batch, int32_t block_size,
                      int32_t *accept_len_out, int32_t *bonus_out, void *stream) {
  if (batch < 0) return DFLASH_ERR_SHAPE;
  if (block_size < 2 || block_size > 64) return DFLASH_ERR_SHAPE;
  if (batch == 0) return DFLASH_OK;
  if (!draft_ids || !target_ids || !accept_len_out || !bonus_out) return DFLASH_ERR_NULL;
  return launch_accept(draft_ids, target_ids, batch, block_size, nullptr, accept_len_out, bonus_out,
                       (hipStream_t)stream) == hipSuccess
             ? DFLASH_OK
             : DFLASH_ERR_HIP;
}

int dflash_accept_len_ragged(const int32_t *draft_ids, const int32_t *target_ids, int32_t batch, int32_t block_size,
                             const int32_t *block_len, int32_t *accept_len_out, int32_t *bonus_out, void *stream) {
  if (batch < 0) return DFLASH_ERR_SHAPE;
  if (block_size < 2 || block_size > 64) return DFLASH_ERR_SHAPE;
  if (batch == 0) return DFLASH_OK;
  if (!draft_ids || !target_ids || !accept_len_out || !bonus_out) return DFLASH_ERR_NULL;
  return launch_accept(draft_ids, target_ids, batch, block_size, block_len, accept_len_out, bonus_out,
                       (hipStream_t)stream) == hipSuccess
             ? DFLASH_OK
             : DFLASH_ERR_HIP;
}

int dflash_check_inputs(dflash_handle h, const dflash_kv *kv, const int32_t *anchor_ids, const int32_t *ids,
                        int32_t n_ids, const int32_t *seq, const int32_t *pos, int32_t n_new, int32_t *err_out,
                        void *stream) {
  if (!h || !err_out) return DFLASH_ERR_NULL;
  int st = validate_kv(h, kv);
  if (st != DFLASH_OK) return st;
  if (n_ids < 0 || n_new < 0) return DFLASH_ERR_SHAPE;
  if ((n_ids > 0 && !ids) || (n_new > 0 && (!seq || !pos))) return DFLASH_ERR_NULL;
  CheckArgs a;
  a.ctx_len = kv->ctx_len;
  a.block_table = kv->block_table;
  a.anchor = anchor_ids;
  a.ids = ids;
  a.seq = seq;
  a.pos = pos;
  a.batch = kv->batch;
  a.max_pages = kv->max_pages;
  a.n_pages = kv->n_pages;
  a.max_ctx = kv->max_ctx;
  a.page_size = h->cfg.page_size;
  a.block_size = h->cfg.block_size;
  a.vocab = h->cfg.vocab;
  a.n_ids = n_ids;
  a.n_new = n_new;
  return launch_check_inputs(a, err_out, (hipStream_t)stream) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

int dflash_sample_workspace_size(int32_t rows, int32_t vocab, size_t *bytes) {
  if (!bytes) return DFLASH_ERR_NULL;
  if (rows < 0 || vocab < 1) return DFLASH_ERR_SHAPE;
  *bytes = sample_ws_bytes(rows, vocab);
  return DFLASH_OK;
}

static bool temperature_ok(float t) { return std::isfinite(t) && t > 0.f && std::isfinite(1.f / t); }

int dflash_sample(const float *logits, int32_t rows, int32_t vocab, float temperature, uint64_t seed,
                  uint32_t offset, uint32_t tag, int32_t *ids_out, float *lse_out, void *ws, size_t ws_bytes,
                  void *stream) {
  if (rows < 0 || vocab < 1) return DFLASH_ERR_SHAPE;
  if (!temperature_ok(temperature) || tag >= 0xFFFFFFFEu) return DFLASH_ERR_RANGE;
  if (rows == 0) return DFLASH_OK;
  if (!logits || !ids_out || !ws) return DFLASH_ERR_NULL;
  if (ws_bytes < sample_ws_bytes(rows, vocab)) return DFLASH_ERR_WORKSPACE;
  return launch_sample(logits, rows, vocab, 1.f / temperature, seed, offset, tag, ids_out, lse_out, ws,
                       (hipStream_t)stream) == hipSuccess
             ? DFLASH_OK
             : DFLASH_ERR_HIP;
}

int dflash_accept_sample(const float *draft_logits, const float *draft_lse, const int32_t *draft_ids,
                         const float *target_logits, const float *target_lse, const int32_t *target_ids,
                         int32_t batch, int32_t block_size, const int32_t *block_len, int32_t vocab,
                         float temperature, uint64_t seed, uint32_t offset, int32_t *accept_len_out,
                         int32_t *bonus_out, void *ws, size_t ws_bytes, void *stream) {
  if (batch < 0 || vocab < 1) return DFLASH_ERR_SHAPE;
  if (block_size < 2 || block_size > 64) return DFLASH_ERR_SHAPE;
  if (!temperature_ok(temperature)) return DFLASH_ERR_RANGE;
  if (batch == 0) return DFLASH_OK;
  if (!draft_logits || !draft_lse || !draft_ids || !target_logits || !target_lse || !target_ids ||
      !accept_len_out || !bonus_out || !ws)
    return DFLASH_ERR_NULL;
  if (ws_bytes < sample_ws_bytes(batch, vocab)) return DFLASH_ERR_WORKSPACE;
  return launch_accept_sample(draft_logits, draft_lse, draft_ids, target_logits, target_lse, target_ids, batch,
                              block_size, block_len, vocab, 1.f / temperature, seed, offset, accept_len_out,
                              bonus_out, ws, (hipStream_t)stream) == hipSuccess
             ? DFLASH_OK
             : DFLASH_ERR_HIP;
}

int dflash_stream_read(const void *src, size_t bytes, uint32_t *sink, void *stream) {
  if (!src || !sink) return DFLASH_ERR_NULL;
  if (bytes % 16 || reinterpret_cast<uintptr_t>(src) % 16) return DFLASH_ERR_SHAPE;
  if (bytes == 0) return DFLASH_OK;
  int dev = 0, n_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || n_cu <= 0)
    n_cu = 256;
  return launch_stream_read(src, bytes, sink, n_cu, (hipStream_t)stream) == hipSuccess ? DFLASH_OK : DFLASH_ERR_HIP;
}

}  // extern "C"
