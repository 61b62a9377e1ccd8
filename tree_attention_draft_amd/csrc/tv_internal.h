// Internal declarations shared by the host glue and the kernel launchers of libtreeverify.
#pragma once
#include <cstdint>

#include <hip/hip_runtime_api.h>

#include "tree_verify.h"

namespace tv {

// Records a detail string for tv_last_error() on this thread and returns `s`.
tv_status fail(tv_status s, const char* detail);

constexpr int kKeysPerTile = 64;  // split chunks are multiples of this many keys
constexpr int kMaxPageSlice = 1024;  // page-table entries one MFMA workgroup stages in LDS
constexpr int kArgSlice = 8192;      // logits of a row per argmax workgroup (one key slot each)
constexpr int kMaxLptBatch = 256;    // largest batch the longest-first request order covers

// Everything a kernel needs, passed by value.  Strides in elements.
struct AttnParams {
  const void* q;
  int64_t q_sb, q_sn, q_sh;
  const void* k;
  const void* v;
  int64_t kv_sb, kv_st, kv_sh;
  const int32_t* page_table;
  int32_t page_size, pages_per_seq, paged;
  int32_t page_shift;  // log2(page_size) when it is a power of two, else -1
  const int32_t* parent;
  int32_t parent_sb;
  const int32_t* prefix_len;
  int32_t max_prefix_len;  // host bound; device values are clamped to [0, this]
  void* out;
  int64_t o_sb, o_sn, o_sh;
  float* lse;
  float* ws_o;    // [B][Hkv][S][R][D] normalised partial outputs (split > 1)
  float* ws_lse;  // [B][Hkv][S][R]    log2-domain partial LSE
  int32_t B, N, Hq, Hkv, g, R;
  int32_t num_splits;  // S
  int32_t chunk;       // keys per split, a multiple of kKeysPerTile
  int32_t row_chunks;  // workgroups along the packed-row dimension (MFMA: head chunks x
                       // node chunks, head chunk fastest)
  int32_t head_chunks; // MFMA: workgroups splitting the group's query heads
  int32_t node_chunks; // MFMA: workgroups splitting each head's 16-node tiles
  int32_t rows_per_wg; // packed rows one workgroup covers
  float scale_log2;    // sm_scale * log2(e)
  int32_t rope;        // fused rotary embedding of q and the tree keys at L + depth
  double rope_log2_theta;
  int32_t lpt;         // MFMA: workgroups take (request, chunk) pieces longest first (ragged)
  int32_t young_from;  // MFMA: workgroups from this linear index on get the higher vector
                       // issue priority (INT32_MAX: none)
  int32_t* meta_depth;     // optional [B, N] copies of the expanded tree (may be null)
  uint64_t* meta_bitmask;
  int32_t* meta_pos;
};

// MFMA kernel shape: `nw` waves per workgroup, one query head each; every wave owns
// `tpw` tiles of 16 tree nodes.  rr = 1: the nodes past those tiles are packed across the
// group's heads into one shared tile that the waves take turns computing.  nc > 1: a
// head's tiles are split over nc workgroups (a wave keeps at most three tiles of state in
// registers), each streaming the same keys.
struct MfmaShape {
  int tpw, nw, rr, nc;
  int teams = 1;  // 2: two teams of nw waves per workgroup (D = 128, nw = 4, no RoPE)
};

// Device-side arguments of the acceptance kernels (argmax over the vocabulary, walk).
struct AcceptParams {
  bool bf16, vec;  // vec: every logits row is 16-byte aligned
  int B, N, V;
  const void* logits;
  int64_t lg_sb, lg_sn;
  const int32_t* tokens;
  int tokens_sb;
  const int32_t* parent;
  int parent_sb;
  int32_t* target;
  int32_t* accepted;
  int32_t* emitted;
  int32_t* num_accepted;
  void* workspace;  // B*N*ceil(V/kArgSlice) uint64 slice keys
};

// Device-side arguments of the stochastic walk kernel.
struct SampleParams {
  bool vec;  // every p and q row is 16-byte aligned
  int B, N, V;
  const float* p;
  int64_t p_sb, p_sn;
  const float* q;
  int64_t q_sb, q_sn;
  const int32_t* tokens;
  int tokens_sb;
  const int32_t* parent;
  int parent_sb;
  const double* uniform;
  int uniform_sb;
  int32_t* accepted;
  int32_t* emitted;
  int32_t* num_accepted;
};

// Device-side arguments of the KV compaction kernel.
struct CompactParams {
  bool bf16, paged;
  int B, N, Hkv, D;
  void* k;
  void* v;
  int64_t kv_sb, kv_st, kv_sh;
  const int32_t* page_table;
  int page_size, pages_per_seq;
  const int32_t* prefix_len;
  int max_prefix_len;
  const int32_t* parent;
  int parent_sb;
  const int32_t* accepted;
  const int32_t* num_accepted;
  int32_t* new_len;
  int32_t* status;
  bool rope;             // write accepted keys rotated at L + j
  double rope_log2_theta;
};

hipError_t launch_argmax(const AcceptParams& p, hipStream_t s);
hipError_t launch_compact(const CompactParams& p, hipStream_t s);
hipError_t launch_stochastic_walk(const SampleParams& p, hipStream_t s);

hipError_t launch_attn_mfma(const AttnParams& p, int D, MfmaShape shape, hipStream_t s);
hipError_t launch_attn_mfma_paged(const AttnParams& p, int D, MfmaShape shape, hipStream_t s);
hipError_t launch_attn_valu(const AttnParams& p, int D, bool bf16, hipStream_t s);
hipError_t launch_merge(const AttnParams& p, int D, bool bf16, hipStream_t s);
hipError_t launch_meta_from_parent(const int32_t* parent, int32_t parent_sb, int32_t B,
                                   int32_t N, const int32_t* prefix_len, int32_t* depth,
                                   uint64_t* bitmask, int32_t* pos, hipStream_t s);

constexpr int kValuRowsPerWg = 16;  // 4 waves x 4 rows

// Where the attention pass finds its split workspace once the plan knows how many bytes it
// needs: the caller's workspace argument, or the library's static device array.
struct WorkspaceSource {
  virtual tv_status get(size_t bytes, void** ptr) const = 0;
 protected:
  ~WorkspaceSource() = default;
};

// The whole pass (checks, plan, launches) with the workspace taken from `ws`.
tv_status attn_pass(const tv_attn_args* a, const WorkspaceSource& ws, hipStream_t stream);

}  // namespace tv
