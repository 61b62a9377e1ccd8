// C-ABI host glue of libtreeverify: argument checks, split planning, kernel dispatch.
// Nothing here allocates device memory or synchronises; every device action is a kernel
// launch on the caller's stream.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdint>
#include <cstring>

#include "tree_verify.h"
#include "tv_internal.h"

namespace tv {

namespace {
thread_local char g_last_error[256] = "";

struct Plan {
  bool mfma = false;
  MfmaShape shape{1, 1};
  int row_chunks = 1;
  int head_chunks = 1;
  int node_chunks = 1;
  int rows_per_wg = 16;
  int splits = 1;
  int chunk = kKeysPerTile;
  bool lpt = false;
  int young_from = INT32_MAX;
  size_t ws_o_bytes = 0;
  size_t ws_bytes = 0;
};

int device_cu_count() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return 256;
  }
  if (dev < 64) {
    const int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0) {
    (void)hipGetLastError();
    n = 256;
  }
  if (dev < 64) cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }

// One wave per query head of the kv head's group (rounded up to a power of two, at most
// 8 waves; larger groups take several head chunks), each wave owning the head's 16-node
// tiles.  When the nodes past the last full tile of all heads fit one 16-row tile (and the
// group is exactly the waves of one workgroup), they are packed into a shared tile that
// the waves take turns computing instead of padding every head's last tile.
MfmaShape pick_mfma_shape(int N, int g, int* head_chunks) {
  int nw = 1;
  while (nw < g && nw < 8) nw *= 2;
  *head_chunks = (g + nw - 1) / nw;
  const int full = N / 16, rem = N % 16;
  if (nw == g && g >= 2 && full >= 1 && full <= 2 && rem > 0 && rem * g <= 16)
    return MfmaShape{full, nw, 1, 1};
  // a wave holds at most three 16-node tiles of state; more are split over node chunks
  const int tiles = (N + 15) / 16;
  const int nc = (tiles + 2) / 3;
  return MfmaShape{(tiles + nc - 1) / nc, nw, 0, nc};
}

tv_status check_args(const tv_attn_args* a, bool pointers) {
  if (!a) return fail(TV_ERR_INVALID_ARG, "args is null");
  if (a->dtype != TV_BF16 && a->dtype != TV_F32) return fail(TV_ERR_INVALID_ARG, "bad dtype");
  if (a->B < 0) return fail(TV_ERR_INVALID_ARG, "B < 0");
  if (a->N < 1) return fail(TV_ERR_INVALID_ARG, "N < 1");
  if (a->N > TV_MAX_NODES) return fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (a->Hq < 1 || a->Hkv < 1 || a->Hq % a->Hkv != 0)
    return fail(TV_ERR_INVALID_ARG, "need Hq >= 1, Hkv >= 1 and Hq % Hkv == 0");
  if (a->D != 64 && a->D != 128) return fail(TV_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (a->kv_layout != TV_KV_CONTIGUOUS && a->kv_layout != TV_KV_PAGED)
    return fail(TV_ERR_INVALID_ARG, "bad kv_layout");
  if (a->path != TV_PATH_AUTO && a->path != TV_PATH_VALU && a->path != TV_PATH_MFMA)
    return fail(TV_ERR_INVALID_ARG, "bad path");
  if (a->path == TV_PATH_MFMA && a->dtype != TV_BF16)
    return fail(TV_ERR_UNSUPPORTED, "the MFMA path takes bf16 inputs");
  if (a->num_splits < 0) return fail(TV_ERR_INVALID_ARG, "num_splits < 0");
  if (a->max_prefix_len < 0 || a->max_prefix_len > INT32_MAX - 2 * TV_MAX_NODES - 64)
    return fail(TV_ERR_INVALID_ARG, "max_prefix_len out of range");
  if (!(a->sm_scale >= 0.f) || !std::isfinite(a->sm_scale))
    return fail(TV_ERR_INVALID_ARG, "sm_scale must be finite and >= 0");
  if (!(a->rope_theta >= 0.0) || !std::isfinite(a->rope_theta))
    return fail(TV_ERR_INVALID_ARG, "rope_theta must be finite and >= 0");
  if (a->B == 0) return TV_OK;
  if (pointers && (!a->q || !a->k || !a->v || !a->parent || !a->prefix_len || !a->out))
    return fail(TV_ERR_INVALID_ARG, "null q, k, v, parent, prefix_len or out");
  if (a->parent_sb < 0) return fail(TV_ERR_INVALID_ARG, "parent_sb < 0");
  if (a->parent_sb > 0 && a->parent_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "parent_sb must be 0 or >= N");
  const int64_t vec = a->dtype == TV_BF16 ? 8 : 4;  // elements per 16 bytes
  const int64_t strides[] = {a->q_sb, a->q_sn, a->q_sh, a->kv_sb, a->kv_st, a->kv_sh,
                             a->o_sb, a->o_sn, a->o_sh};
  for (int64_t s : strides) {
    if (s < 0 || s % vec != 0)
      return fail(TV_ERR_INVALID_ARG, "strides must be >= 0 and multiples of 16 bytes");
  }
  if (pointers &&
      (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->out)))
    return fail(TV_ERR_INVALID_ARG, "q, k, v and out must be 16-byte aligned");
  if (a->kv_layout == TV_KV_PAGED) {
    if ((pointers && !a->page_table) || a->page_size < 1 || a->pages_per_seq < 1)
      return fail(TV_ERR_INVALID_ARG, "paged KV needs page_table, page_size, pages_per_seq");
    const int64_t need = ((int64_t)a->max_prefix_len + a->N + a->page_size - 1) / a->page_size;
    if (a->pages_per_seq < need)
      return fail(TV_ERR_INVALID_ARG, "pages_per_seq too small for max_prefix_len + N");
  }
  if (a->B > 65535) return fail(TV_ERR_UNSUPPORTED, "B > 65535");
  return TV_OK;
}

tv_status make_plan(const tv_attn_args* a, Plan* pl) {
  const int g = a->Hq / a->Hkv;
  const int R = a->N * g;
  const bool bf16 = a->dtype == TV_BF16;
  pl->mfma = a->path == TV_PATH_MFMA || (a->path == TV_PATH_AUTO && bf16 && R >= 16);
  if (pl->mfma) {
    pl->shape = pick_mfma_shape(a->N, g, &pl->head_chunks);
    pl->node_chunks = pl->shape.nc;
    pl->row_chunks = pl->head_chunks * pl->node_chunks;
    pl->rows_per_wg = pl->shape.nw * a->N;
  } else {
    pl->rows_per_wg = kValuRowsPerWg;
    pl->row_chunks = (R + kValuRowsPerWg - 1) / kValuRowsPerWg;
    pl->head_chunks = pl->row_chunks;
    pl->node_chunks = 1;
  }
  if ((int64_t)a->Hkv * pl->row_chunks > 65535)
    return fail(TV_ERR_UNSUPPORTED, "Hkv * row chunks > 65535");
  const int64_t tmax = (int64_t)a->max_prefix_len + a->N;
  const int64_t tiles = (tmax + kKeysPerTile - 1) / kKeysPerTile;  // every request fits
  // Key tiles of the whole batch: from the host copy of the prefix lengths when the caller
  // gives one, else as if every request had max_prefix_len.
  int64_t work = 0;
  bool ragged = false;
  for (int b = 0; b < a->B; ++b) {
    const int64_t Lb = a->prefix_len_host
        ? std::min<int64_t>(std::max<int32_t>(a->prefix_len_host[b], 0), a->max_prefix_len)
        : a->max_prefix_len;
    work += (Lb + a->N + kKeysPerTile - 1) / kKeysPerTile;
    if (a->prefix_len_host && a->prefix_len_host[b] != a->prefix_len_host[0]) ragged = true;
  }
  const int64_t pair_tiles = work * a->Hkv * pl->row_chunks;
  int64_t S;
  if (a->num_splits > 0) {
    S = std::min<int64_t>(a->num_splits, tiles);
  } else {
    // chunks of the batch's average work per workgroup slot (two per compute unit): a
    // batch of equal requests that fills the slots keeps one split, smaller ones split
    // until they fill them.  A ragged batch (lengths known from the host copy) is cut the
    // same way, its pieces then taken longest first (on MI355X, L ~ U[512, 8192], back to
    // back: B=64 246.9 us against 255.2 us with chunks of two thirds of the average, B=32
    // 132.3 against 139.2 us; after an idle GPU, where the clock is cut, 315.5 against
    // 317.2 us)
    // When that leaves a workgroup under 8 chunk units of 64 keys (small batches), chunks
    // are sized for one workgroup per compute unit instead: each workgroup pays a prologue
    // and a partial of R*(D+1)*4 bytes, which short chunks cannot hide (MI355X, L=2048,
    // B=8: 24.5 us at 4 splits against 25.7 at 6 and 25.9 at 8; paged L=32768, B=1, nine
    // units a workgroup at two per unit: 59.4 us at 57 splits against 65.6 at 31).
    // Slots: two workgroups per compute unit, one for the eight-wave shapes (their register
    // use allows two waves per SIMD, i.e. eight waves per unit; B=16,
    // N=64, 64q/8kv: 152 us with one split against 183 us with the two that two slots
    // per unit would ask for).
    const int64_t cus = device_cu_count();
    const int64_t per_cu = pl->mfma && pl->shape.nw >= 8 ? 1 : 2;
    int64_t avg = (pair_tiles + per_cu * cus - 1) / (per_cu * cus);
    if (avg < 8) avg = (pair_tiles + cus - 1) / cus;
    const int64_t chunk_tiles = std::max<int64_t>(1, avg);
    S = (tiles + chunk_tiles - 1) / chunk_tiles;
  }
  S = std::max<int64_t>(S, 1);
  pl->lpt = pl->mfma && ragged && a->B <= kMaxLptBatch;
  if (pl->mfma && a->kv_layout == TV_KV_PAGED) {
    // a split's page-table slice must fit the kernel's LDS copy
    const int64_t max_keys = (int64_t)(kMaxPageSlice - 1) * a->page_size;
    const int64_t max_tiles = std::max<int64_t>(1, max_keys / kKeysPerTile);
    S = std::max<int64_t>(S, (tiles + max_tiles - 1) / max_tiles);
  }
  const int64_t chunk_tiles = (tiles + S - 1) / S;
  S = (tiles + chunk_tiles - 1) / chunk_tiles;
  pl->splits = (int)S;
  pl->chunk = (int)(chunk_tiles * kKeysPerTile);
  // A grid of exactly two four-wave workgroups per compute unit is dispatched breadth
  // first: workgroup i and workgroup i + CUs share a unit, and the older one wins issue
  // ties and finishes ~15% earlier, leaving its partner alone for the tail.  The younger
  // ones get the higher priority for their vector phases (B=64, L=4096, N=33: -4%).
  if (pl->mfma && pl->shape.nw == 4 && pl->shape.tpw <= 2 && !pl->lpt) {
    const int64_t cus = device_cu_count();
    if (S * a->Hkv * pl->row_chunks * (int64_t)a->B == 2 * cus) pl->young_from = (int)cus;
  }
  // A grid of at most one workgroup per compute unit (small batches) would leave each SIMD
  // a single wave: the four-wave shapes then run two teams of four waves per workgroup,
  // splitting every window's tiles (D = 128, no fused rotary embedding).
  if (pl->mfma && a->D == 128 && !(a->rope_theta > 0.0) && pl->shape.nw == 4) {
    const int64_t wgs = S * a->Hkv * pl->row_chunks * (int64_t)a->B;
    if (wgs <= device_cu_count()) pl->shape.teams = 2;
  }
  if (S > 1) {
    const size_t rows = (size_t)a->B * a->Hkv * S * R;
    pl->ws_o_bytes = rows * a->D * sizeof(float);
    pl->ws_bytes = pl->ws_o_bytes + rows * sizeof(float);
  }
  return TV_OK;
}

AttnParams make_params(const tv_attn_args* a, const Plan& pl, void* workspace) {
  AttnParams p{};
  p.q = a->q;
  p.q_sb = a->q_sb;
  p.q_sn = a->q_sn;
  p.q_sh = a->q_sh;
  p.k = a->k;
  p.v = a->v;
  p.kv_sb = a->kv_sb;
  p.kv_st = a->kv_st;
  p.kv_sh = a->kv_sh;
  p.paged = a->kv_layout == TV_KV_PAGED;
  p.page_table = a->page_table;
  p.page_size = p.paged ? a->page_size : 1;
  p.pages_per_seq = a->pages_per_seq;
  p.page_shift = -1;
  if (p.paged && (a->page_size & (a->page_size - 1)) == 0) {
    int sh = 0;
    while ((1 << sh) < a->page_size) ++sh;
    p.page_shift = sh;
  }
  p.parent = a->parent;
  p.parent_sb = a->parent_sb;
  p.prefix_len = a->prefix_len;
  p.max_prefix_len = a->max_prefix_len;
  p.out = a->out;
  p.o_sb = a->o_sb;
  p.o_sn = a->o_sn;
  p.o_sh = a->o_sh;
  p.lse = a->lse;
  p.B = a->B;
  p.N = a->N;
  p.Hq = a->Hq;
  p.Hkv = a->Hkv;
  p.g = a->Hq / a->Hkv;
  p.R = a->N * p.g;
  p.num_splits = pl.splits;
  p.chunk = pl.chunk;
  p.row_chunks = pl.row_chunks;
  p.head_chunks = pl.head_chunks;
  p.node_chunks = pl.node_chunks;
  p.rows_per_wg = pl.rows_per_wg;
  const float scale = a->sm_scale > 0.f ? a->sm_scale : 1.0f / std::sqrt((float)a->D);
  p.scale_log2 = scale * 1.4426950408889634f;
  p.rope = a->rope_theta > 0.0;
  p.rope_log2_theta = p.rope ? std::log2(a->rope_theta) : 0.0;
  p.lpt = pl.lpt ? 1 : 0;
  p.young_from = pl.young_from;
  p.meta_depth = a->meta_depth;
  p.meta_bitmask = a->meta_bitmask;
  p.meta_pos = a->meta_pos;
  if (pl.splits > 1) {
    p.ws_o = static_cast<float*>(workspace);
    p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + pl.ws_o_bytes);
  }
  return p;
}

}  // namespace

tv_status fail(tv_status s, const char* detail) {
  std::strncpy(g_last_error, detail ? detail : "", sizeof(g_last_error) - 1);
  g_last_error[sizeof(g_last_error) - 1] = '\0';
  return s;
}

}  // namespace tv

using namespace tv;

extern "C" size_t tree_verify_attn_workspace_size(const tv_attn_args* a) {
  if (check_args(a, false) != TV_OK || a->B == 0) return 0;
  Plan pl;
  if (make_plan(a, &pl) != TV_OK) return 0;
  return pl.ws_bytes;
}

namespace tv {

tv_status attn_pass(const tv_attn_args* a, const WorkspaceSource& ws, hipStream_t stream) {
  tv_status st = check_args(a, true);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  Plan pl;
  st = make_plan(a, &pl);
  if (st != TV_OK) return st;
  void* workspace = nullptr;
  if (pl.ws_bytes > 0) {
    st = ws.get(pl.ws_bytes, &workspace);
    if (st != TV_OK) return st;
    if (!aligned16(workspace)) return fail(TV_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  }
  const AttnParams p = make_params(a, pl, workspace);
  const bool bf16 = a->dtype == TV_BF16;
  hipError_t e = pl.mfma ? launch_attn_mfma(p, a->D, pl.shape, stream)
                         : launch_attn_valu(p, a->D, bf16, stream);
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  if (pl.splits > 1) {
    e = launch_merge(p, a->D, bf16, stream);
    if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  }
  return TV_OK;
}

}  // namespace tv

namespace {

// The caller's workspace argument.
struct CallerWorkspace final : tv::WorkspaceSource {
  const tv_attn_args* a;
  explicit CallerWorkspace(const tv_attn_args* args) : a(args) {}
  tv_status get(size_t bytes, void** ptr) const override {
    if (!a->workspace || a->workspace_bytes < bytes)
      return tv::fail(TV_ERR_WORKSPACE, "workspace missing or smaller than required");
    *ptr = a->workspace;
    return TV_OK;
  }
};

}  // namespace

extern "C" tv_status tree_verify_attn(const tv_attn_args* a, hipStream_t stream) {
  return tv::attn_pass(a, CallerWorkspace(a), stream);
}

extern "C" tv_status tree_meta_from_parent(const int32_t* parent, int32_t parent_sb, int32_t B,
                                           int32_t N, const int32_t* prefix_len,
                                           int32_t* depth, uint64_t* bitmask, int32_t* pos,
                                           hipStream_t stream) {
  if (B < 0) return fail(TV_ERR_INVALID_ARG, "B < 0");
  if (N < 1) return fail(TV_ERR_INVALID_ARG, "N < 1");
  if (N > TV_MAX_NODES) return fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (parent_sb < 0 || (parent_sb > 0 && parent_sb < N))
    return fail(TV_ERR_INVALID_ARG, "parent_sb must be 0 or >= N");
  if (B == 0) return TV_OK;
  if (!parent) return fail(TV_ERR_INVALID_ARG, "parent is null");
  const hipError_t e =
      launch_meta_from_parent(parent, parent_sb, B, N, prefix_len, depth, bitmask, pos, stream);
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  return TV_OK;
}

// ---------------------------------------------------------------- acceptance -------
namespace tv {
namespace {

tv_status check_accept(const tv_accept_args* a) {
  if (!a) return fail(TV_ERR_INVALID_ARG, "args is null");
  if (a->dtype != TV_BF16 && a->dtype != TV_F32) return fail(TV_ERR_INVALID_ARG, "bad dtype");
  if (a->B < 0) return fail(TV_ERR_INVALID_ARG, "B < 0");
  if (a->N < 1) return fail(TV_ERR_INVALID_ARG, "N < 1");
  if (a->N > TV_MAX_NODES) return fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (a->V < 1) return fail(TV_ERR_INVALID_ARG, "V < 1");
  if (a->B == 0) return TV_OK;
  if (!a->logits || !a->tokens || !a->parent || !a->target || !a->accepted || !a->emitted ||
      !a->num_accepted)
    return fail(TV_ERR_INVALID_ARG, "null pointer argument");
  if (a->lg_sn < a->V || a->lg_sb < 0 || (a->B > 1 && a->lg_sb < (int64_t)a->N * a->lg_sn))
    return fail(TV_ERR_INVALID_ARG, "logits strides must cover [B, N, V] without overlap");
  if (a->tokens_sb != 0 && a->tokens_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "tokens_sb must be 0 or >= N");
  if (a->parent_sb != 0 && a->parent_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "parent_sb must be 0 or >= N");
  const uintptr_t esz = a->dtype == TV_BF16 ? 2 : 4;
  if (reinterpret_cast<uintptr_t>(a->logits) % esz != 0)
    return fail(TV_ERR_INVALID_ARG, "logits not aligned to its element size");
  if (a->V > (1 << 30)) return fail(TV_ERR_INVALID_ARG, "V > 2^30");
  if ((int64_t)a->B * a->N > 65535) return fail(TV_ERR_UNSUPPORTED, "B * N > 65535");
  const size_t need = tree_accept_greedy_workspace_size(a);
  if (!a->workspace || a->workspace_bytes < need)
    return fail(TV_ERR_WORKSPACE, "workspace missing or smaller than required");
  if (!aligned16(a->workspace)) return fail(TV_ERR_INVALID_ARG, "workspace not 16-byte aligned");
  return TV_OK;
}

tv_status check_sample(const tv_sample_args* a) {
  if (!a) return fail(TV_ERR_INVALID_ARG, "args is null");
  if (a->B < 0) return fail(TV_ERR_INVALID_ARG, "B < 0");
  if (a->N < 1) return fail(TV_ERR_INVALID_ARG, "N < 1");
  if (a->N > TV_MAX_NODES) return fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (a->V < 1) return fail(TV_ERR_INVALID_ARG, "V < 1");
  if (a->V > (1 << 30)) return fail(TV_ERR_INVALID_ARG, "V > 2^30");
  if (a->B == 0) return TV_OK;
  if (!a->p || !a->q || !a->tokens || !a->parent || !a->uniform || !a->accepted ||
      !a->emitted || !a->num_accepted)
    return fail(TV_ERR_INVALID_ARG, "null pointer argument");
  const int64_t rows[][2] = {{a->p_sb, a->p_sn}, {a->q_sb, a->q_sn}};
  for (const auto& r : rows)
    if (r[1] < a->V || r[0] < 0 || (a->B > 1 && r[0] < (int64_t)a->N * r[1]))
      return fail(TV_ERR_INVALID_ARG, "p and q strides must cover [B, N, V] without overlap");
  if (a->tokens_sb != 0 && a->tokens_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "tokens_sb must be 0 or >= N");
  if (a->parent_sb != 0 && a->parent_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "parent_sb must be 0 or >= N");
  if (a->uniform_sb != 0 && a->uniform_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "uniform_sb must be 0 or >= N");
  if ((reinterpret_cast<uintptr_t>(a->p) | reinterpret_cast<uintptr_t>(a->q)) % 4 != 0 ||
      reinterpret_cast<uintptr_t>(a->uniform) % 8 != 0)
    return fail(TV_ERR_INVALID_ARG, "p, q or uniform not aligned to its element size");
  if (a->B > 65535) return fail(TV_ERR_UNSUPPORTED, "B > 65535");
  return TV_OK;
}

tv_status check_compact(const tv_compact_args* a) {
  if (!a) return fail(TV_ERR_INVALID_ARG, "args is null");
  if (a->dtype != TV_BF16 && a->dtype != TV_F32) return fail(TV_ERR_INVALID_ARG, "bad dtype");
  if (a->B < 0) return fail(TV_ERR_INVALID_ARG, "B < 0");
  if (a->N < 1) return fail(TV_ERR_INVALID_ARG, "N < 1");
  if (a->N > TV_MAX_NODES) return fail(TV_ERR_UNSUPPORTED, "N > 64");
  if (a->Hkv < 1) return fail(TV_ERR_INVALID_ARG, "Hkv < 1");
  if (a->D != 64 && a->D != 128) return fail(TV_ERR_UNSUPPORTED, "D must be 64 or 128");
  if (a->kv_layout != TV_KV_CONTIGUOUS && a->kv_layout != TV_KV_PAGED)
    return fail(TV_ERR_INVALID_ARG, "bad kv_layout");
  if (a->max_prefix_len < 0 || a->max_prefix_len > (1 << 30))
    return fail(TV_ERR_INVALID_ARG, "max_prefix_len out of range");
  if (!(a->rope_theta >= 0.0) || !std::isfinite(a->rope_theta))
    return fail(TV_ERR_INVALID_ARG, "rope_theta must be finite and >= 0");
  if (a->B == 0) return TV_OK;
  if (!a->k || !a->v || !a->prefix_len || !a->parent || !a->accepted || !a->num_accepted)
    return fail(TV_ERR_INVALID_ARG, "null pointer argument");
  if (a->parent_sb != 0 && a->parent_sb < a->N)
    return fail(TV_ERR_INVALID_ARG, "parent_sb must be 0 or >= N");
  const int64_t vec = a->dtype == TV_BF16 ? 8 : 4;
  const int64_t strides[] = {a->kv_sb, a->kv_st, a->kv_sh};
  for (int64_t st : strides)
    if (st < 0 || st % vec != 0)
      return fail(TV_ERR_INVALID_ARG, "strides must be >= 0 and multiples of 16 bytes");
  if (!aligned16(a->k) || !aligned16(a->v))
    return fail(TV_ERR_INVALID_ARG, "k and v must be 16-byte aligned");
  if (a->kv_layout == TV_KV_PAGED) {
    if (!a->page_table || a->page_size < 1 || a->pages_per_seq < 1)
      return fail(TV_ERR_INVALID_ARG, "paged KV needs page_table, page_size, pages_per_seq");
    const int64_t need = ((int64_t)a->max_prefix_len + a->N + a->page_size - 1) / a->page_size;
    if (a->pages_per_seq < need)
      return fail(TV_ERR_INVALID_ARG, "pages_per_seq too small for max_prefix_len + N");
  }
  return TV_OK;
}

}  // namespace
}  // namespace tv

extern "C" tv_status tree_accept_greedy(const tv_accept_args* a, hipStream_t stream) {
  using namespace tv;
  tv_status st = check_accept(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  AcceptParams p;
  p.bf16 = a->dtype == TV_BF16;
  const int64_t esz = p.bf16 ? 2 : 4;
  p.vec = aligned16(a->logits) && (a->lg_sb * esz) % 16 == 0 && (a->lg_sn * esz) % 16 == 0;
  p.B = a->B;
  p.N = a->N;
  p.V = a->V;
  p.logits = a->logits;
  p.lg_sb = a->lg_sb;
  p.lg_sn = a->lg_sn;
  p.tokens = a->tokens;
  p.tokens_sb = a->tokens_sb;
  p.parent = a->parent;
  p.parent_sb = a->parent_sb;
  p.target = a->target;
  p.accepted = a->accepted;
  p.emitted = a->emitted;
  p.num_accepted = a->num_accepted;
  p.workspace = a->workspace;
  const hipError_t e = launch_argmax(p, stream);
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  return TV_OK;
}

extern "C" tv_status tree_accept_stochastic(const tv_sample_args* a, hipStream_t stream) {
  using namespace tv;
  tv_status st = check_sample(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  SampleParams p;
  p.vec = aligned16(a->p) && aligned16(a->q) && a->p_sb % 4 == 0 && a->p_sn % 4 == 0 &&
          a->q_sb % 4 == 0 && a->q_sn % 4 == 0;
  p.B = a->B;
  p.N = a->N;
  p.V = a->V;
  p.p = a->p;
  p.p_sb = a->p_sb;
  p.p_sn = a->p_sn;
  p.q = a->q;
  p.q_sb = a->q_sb;
  p.q_sn = a->q_sn;
  p.tokens = a->tokens;
  p.tokens_sb = a->tokens_sb;
  p.parent = a->parent;
  p.parent_sb = a->parent_sb;
  p.uniform = a->uniform;
  p.uniform_sb = a->uniform_sb;
  p.accepted = a->accepted;
  p.emitted = a->emitted;
  p.num_accepted = a->num_accepted;
  const hipError_t e = launch_stochastic_walk(p, stream);
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  return TV_OK;
}

extern "C" tv_status tree_kv_compact(const tv_compact_args* a, hipStream_t stream) {
  using namespace tv;
  tv_status st = check_compact(a);
  if (st != TV_OK) return st;
  if (a->B == 0) return TV_OK;
  CompactParams p;
  p.bf16 = a->dtype == TV_BF16;
  p.paged = a->kv_layout == TV_KV_PAGED;
  p.B = a->B;
  p.N = a->N;
  p.Hkv = a->Hkv;
  p.D = a->D;
  p.k = a->k;
  p.v = a->v;
  p.kv_sb = a->kv_sb;
  p.kv_st = a->kv_st;
  p.kv_sh = a->kv_sh;
  p.page_table = a->page_table;
  p.page_size = a->page_size;
  p.pages_per_seq = a->pages_per_seq;
  p.prefix_len = a->prefix_len;
  p.max_prefix_len = a->max_prefix_len;
  p.parent = a->parent;
  p.parent_sb = a->parent_sb;
  p.accepted = a->accepted;
  p.num_accepted = a->num_accepted;
  p.new_len = a->new_len;
  p.status = a->status;
  p.rope = a->rope_theta > 0.0;
  p.rope_log2_theta = p.rope ? std::log2(a->rope_theta) : 0.0;
  const hipError_t e = launch_compact(p, stream);
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  return TV_OK;
}

extern "C" size_t tree_accept_greedy_workspace_size(const tv_accept_args* a) {
  if (!a || a->B < 0 || a->N < 1 || a->N > TV_MAX_NODES || a->V < 1) return 0;
  const size_t slices = ((size_t)a->V + tv::kArgSlice - 1) / tv::kArgSlice;
  return (size_t)a->B * a->N * slices * 8;
}

extern "C" size_t tv_accept_args_sizeof(void) { return sizeof(tv_accept_args); }
extern "C" size_t tv_sample_args_sizeof(void) { return sizeof(tv_sample_args); }
extern "C" size_t tv_compact_args_sizeof(void) { return sizeof(tv_compact_args); }

extern "C" const char* tv_status_string(tv_status s) {
  switch (s) {
    case TV_OK: return "TV_OK";
    case TV_ERR_INVALID_ARG: return "TV_ERR_INVALID_ARG";
    case TV_ERR_INVALID_PATH: return "TV_ERR_INVALID_PATH";
    case TV_ERR_MISSING_PARENT: return "TV_ERR_MISSING_PARENT";
    case TV_ERR_CAPACITY: return "TV_ERR_CAPACITY";
    case TV_ERR_UNSUPPORTED: return "TV_ERR_UNSUPPORTED";
    case TV_ERR_WORKSPACE: return "TV_ERR_WORKSPACE";
    case TV_ERR_HIP: return "TV_ERR_HIP";
  }
  return "TV_ERR_UNKNOWN";
}

extern "C" const char* tv_last_error(void) { return g_last_error; }

extern "C" tv_status tv_pinned_device_address(const void* host, const void** device) {
  if (!host || !device) return fail(TV_ERR_INVALID_ARG, "null argument");
  void* d = nullptr;
  const hipError_t e = hipHostGetDevicePointer(&d, const_cast<void*>(host), 0);
  *device = e == hipSuccess ? d : nullptr;
  if (e != hipSuccess) return fail(TV_ERR_HIP, hipGetErrorString(e));
  return TV_OK;
}

extern "C" int32_t tv_abi_version(void) { return TV_ABI_VERSION; }

extern "C" size_t tv_attn_args_sizeof(void) { return sizeof(tv_attn_args); }
