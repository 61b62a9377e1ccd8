// Tree-verify attention, MFMA path (bf16 inputs, fp32 accumulation, gfx950).
//
// Semantics ("Tree attention mask for draft-tree verification", "A strong answer";
// "Tree Verification", "Tree Attention"): query head j of the kv head's group, at tree node
// i, attends every prefix key t < L and tree key L + a exactly when a is i or an ancestor
// of i.  The ancestor bitmask is built in LDS from the parent array once per workgroup
// and turned into one 64-bit "allowed" word per row per key tile; tiles that hold only
// prefix keys carry no mask at all.
//
// Work decomposition.  One workgroup = (key split, kv head x head chunk x node chunk,
// request) with NW waves; wave w owns query head j = chunk*NW + w of the group and TN of
// its 16-node tiles (all of them unless long trees are split over node chunks), so every
// wave does the same amount of work; the nodes past the last full tile of all heads can
// share one tile that the waves take turns computing (RR, below).  Each 32-key tile of K
// and V is read from HBM once per workgroup and reused by every head and node of it.
//
// Memory pipeline.  K and V tiles are copied global -> LDS by direct loads
// (global_load_lds, 16 bytes per lane) into an NST-stage ring holding two windows of NST/2
// tiles: no registers are tied up in flight.  One barrier per window publishes its tiles
// and frees the previous window's stages, into which the next window's loads are issued
// right away, so they stream while this window is computed.  LDS rows are XOR-swizzled
// per 16-byte chunk (K by row, V by row pairs; see swz_k / swz_v) so operand reads are
// conflict-free.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16; lane l, lr = l % 16, lh = l / 16):
//   A operand: row lr, k = 8*lh .. 8*lh+7;  B operand: column lr, same k;
//   result:    rows 4*lh .. 4*lh+3 of column lr.
// Scores are computed transposed, S^T = K Q^T (A = K from LDS, B = Q in registers): a lane
// holds 4 keys of ONE query row, so the row max is in-lane plus two cross-lane steps and
// the row sum stays per lane until the end.  The output is accumulated transposed too,
// O^T += V^T P^T: the P values a lane owns (keys 4lh..4lh+3 of two 16-key blocks) form a
// B operand once the contraction index is permuted the same way on both sides, so P never
// leaves registers.  The matching A operand (V^T) comes straight from V's natural
// row-major layout through the transposing LDS read ds_read_b64_tr_b16: within each
// 16-lane group, lane s addresses V[base + s/4][d0 + 4*(s%4) ..] and output lane l receives
// V[base + j][d0 + l] for j = 0..3.
#pragma once
// The kernel template is instantiated twice: for contiguous KV (attn_mfma.hip) and for
// paged KV (attn_mfma_paged.hip), so that each form carries only its own address code
// and registers; the two translation units build in parallel.
#include <type_traits>

#include "mfma_common.h"

namespace tv {

// Wave issue priority around a block of matrix instructions: the two waves sharing a SIMD
// mostly alternate between matrix and vector work; letting the wave that is issuing MFMAs
// go first keeps the matrix pipe fed while the other fills the gaps with its vector work.
// The scheduling barriers keep the compiler from moving instructions across the change.
// `young`: this workgroup shares its compute unit with an older one that would otherwise
// win every tie; its vector phases then outrank the older one's (matrix phases still
// outrank both).
__device__ inline void mfma_priority(bool high, bool young) {
  __builtin_amdgcn_sched_barrier(0);
  if (high)
    __builtin_amdgcn_s_setprio(2);
  else if (young)
    __builtin_amdgcn_s_setprio(1);
  else
    __builtin_amdgcn_s_setprio(0);
  __builtin_amdgcn_sched_barrier(0);
}

template <int D, int KT, int NST, int TN, int NW>
struct MfmaCfg {
  static constexpr int DS = D / 32;             // k-steps of Q.K^T
  static constexpr int DB = D / 16;             // 16-feature output blocks
  static constexpr int ROWB = D * 2;            // bytes per K or V row
  static constexpr int CH = D / 8;              // 16-byte chunks per row
  static constexpr int TILEB = KT * ROWB;       // bytes of one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;      // K tile then V tile
  static constexpr int RPI = 1024 / ROWB;       // rows per 1 KB load instruction
  static constexpr int LI = STAGEB / 1024;      // load instructions per tile
  static constexpr int LPW = LI / NW;           // ... per wave
  static constexpr int KB = KT / 16;            // 16-key blocks per tile
  static constexpr int KS = KT / 32;            // 32-key steps of P.V
  static_assert(LI % NW == 0, "load instructions must split evenly over the waves");
  static_assert(KT % 32 == 0 && NST >= 2, "tile shape");
};

// XOR swizzles of the 16-byte chunk index, period = the whole row (CH chunks): K rows by
// row mod CH, so the 16-byte operand reads of any 16 consecutive rows hit distinct banks;
// V rows by 2*(row mod CH/2), so the 32-byte transposed-read segments of any 8
// consecutive rows do.
template <int CH>
__device__ inline int swz_k(int r) { return r & (CH - 1); }
template <int CH>
__device__ inline int swz_v(int r) { return (r & (CH / 2 - 1)) << 1; }

// Per-wave load assignment.  When a wave has an even number LPW of 1 KB load instructions
// per tile, its first LPW/2 copy K and the others V (known at compile time); K (V)
// instruction jj of wave w covers rows (jj*NW + w)*RPI ... of its tile.  Otherwise
// (LPW = 1) instruction i = w of the tile's LI copies K when i < LI/2, else V.  For each
// instruction a lane owns one 16-byte chunk: row r, LDS position lane % CH, global chunk
// swizzled.
template <class C, int NW>
struct LoadPlan {
  static constexpr bool kSplit = C::LPW % 2 == 0;
  static constexpr int HALF = kSplit ? C::LPW / 2 : 1;
  static_assert(kSplit || C::LPW == 1, "load instructions per wave");
  bool v1;               // LPW = 1: this wave copies V (wave-uniform)
  uint32_t dst0;         // LDS byte offset of the wave's first K (or only) instruction
  uint32_t off[C::LPW];  // contiguous KV: byte offset of the chunk from the tile's row 0

  __device__ inline bool is_v(int ii) const { return kSplit ? ii >= HALF : v1; }
  // row within the tile and byte offset of the (swizzled) global chunk within the row
  __device__ inline void chunk_of(int ii, int w, int lane, int& r, int& coff) const {
    const bool v = is_v(ii);
    const int ik = kSplit ? (ii % HALF) * NW + w : (v ? w - C::LI / 2 : w);
    r = ik * C::RPI + lane / C::CH;
    coff = ((lane % C::CH) ^ (v ? swz_v<C::CH>(r) : swz_k<C::CH>(r))) * 16;
  }
  // first tile row that instruction ii of wave w copies (wave-uniform)
  __device__ inline int first_row(int ii, int w) const {
    const int ik = kSplit ? (ii % HALF) * NW + w : (is_v(ii) ? w - C::LI / 2 : w);
    return ik * C::RPI;
  }
  // LDS byte offset of instruction ii within a stage
  __device__ inline uint32_t dst(int ii) const {
    if constexpr (kSplit) return dst0 + (ii >= HALF ? C::TILEB : 0) + (ii % HALF) * NW * 1024;
    return dst0;
  }

  __device__ LoadPlan(const AttnParams& p, int w, int lane) {
    v1 = !kSplit && w >= C::LI / 2;
    dst0 = kSplit ? w * 1024 : (v1 ? C::TILEB + (w - C::LI / 2) * 1024 : w * 1024);
#pragma unroll
    for (int ii = 0; ii < C::LPW; ++ii) {
      int r, coff;
      chunk_of(ii, w, lane, r, coff);
      off[ii] = (uint32_t)((int64_t)r * p.kv_st * 2 + coff);
    }
  }
};

// Issue the direct loads of the tile at logical key kt0 into the stage at LDS address
// `stage`.  Full tiles of contiguous KV (`fast`: the per-lane offsets fit 32 bits) use a
// scalar tile base plus the precomputed lane offsets.  Full tiles of paged KV whose pages
// hold a whole number of one instruction's rows (`pfast`: page size a power of two and a
// multiple of RPI) do the same with one page lookup per instruction: the RPI rows an
// instruction copies lie in one page, so its base is wave-uniform.  Otherwise (the last,
// partial tile, or other page sizes) rows at or past kend are redirected to key kend-1
// (finite data, masked out later), so every LDS slot of the stage is rewritten and no read
// leaves [0, kend).
template <class C, int NW, int KT, bool VA>
__device__ inline void issue_tile(const AttnParams& p, const RowMap& rm,
                                  const LoadPlan<C, NW>& lp, const char* kg, const char* vg,
                                  uint32_t stage, int kt0, int kend, bool fast, bool pfast,
                                  int w, int lane) {
  if (fast && kt0 + KT <= kend) {
    const int64_t row0 = (rm.head_off + (int64_t)kt0 * p.kv_st) * 2;
    const char* kb = kg + row0;
    const char* vb = vg + row0;
#pragma unroll
    for (int ii = 0; ii < C::LPW; ++ii)
      lds_load16_s(lp.is_v(ii) ? vb : kb, lp.off[ii], stage + lp.dst(ii));
    return;
  }
  if (pfast && kt0 + KT <= kend && !VA) {
    // one LDS read for all of the wave's instructions: lane i fetches instruction i's page
    const int li = lane < C::LPW ? lane : 0;
    const int lpage = rm.pt[((kt0 + lp.first_row(li, w)) >> p.page_shift) - rm.pbase];
#pragma unroll
    for (int ii = 0; ii < C::LPW; ++ii) {
      const int r0 = lp.first_row(ii, w);
      const int t0 = kt0 + r0;
      const int page = __builtin_amdgcn_readlane(lpage, ii);
      // element offset of tile row 0 as if the page continued backwards: lp.off holds the
      // lane's row r0 + lane/CH relative to row 0
      const int64_t el = (int64_t)page * p.kv_sb + rm.head_off +
                         (int64_t)((t0 & (p.page_size - 1)) - r0) * p.kv_st;
      lds_load16_s((lp.is_v(ii) ? vg : kg) + el * 2, lp.off[ii], stage + lp.dst(ii));
    }
    return;
  }
  if (pfast && kt0 + KT <= kend) {
    // VA (paged instantiations with registers to spare): lane i (< LPW) forms the base
    // address of the wave's instruction i, so one LDS read of page ids and one 64-bit
    // address computation on the vector unit serve every instruction, each then taking its
    // base with two readlanes (a scalar multiply chain per instruction, as above, costs
    // about a twentieth of the paged pass).  The base is that of tile row 0 as if the page
    // continued backwards.
    const int li = lane < C::LPW ? lane : 0;
    const int r0 = lp.first_row(li, w);
    const int t0 = kt0 + r0;
    const int page = rm.pt[(t0 >> p.page_shift) - rm.pbase];
    const int64_t el = (int64_t)page * p.kv_sb + rm.head_off +
                       (int64_t)((t0 & (p.page_size - 1)) - r0) * p.kv_st;
    const uint64_t addr = (uint64_t)(uintptr_t)((lp.is_v(li) ? vg : kg) + el * 2);
    const int alo = (int)(uint32_t)addr, ahi = (int)(uint32_t)(addr >> 32);
#pragma unroll
    for (int ii = 0; ii < C::LPW; ++ii) {
      const uint64_t a = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane(ahi, ii) << 32) |
                         (uint32_t)__builtin_amdgcn_readlane(alo, ii);
      lds_load16_s(reinterpret_cast<const char*>((uintptr_t)a), lp.off[ii], stage + lp.dst(ii));
    }
    return;
  }
#pragma unroll
  for (int ii = 0; ii < C::LPW; ++ii) {
    int r, coff;
    lp.chunk_of(ii, w, lane, r, coff);
    const int t = min(kt0 + r, kend - 1);
    const char* src = (lp.is_v(ii) ? vg : kg) + row_offset(p, rm, t) * 2 + coff;
    lds_load16(src, stage + lp.dst(ii));
  }
}

// Online softmax of one 16-row x KT-key score tile held transposed (lane: 4 keys of one
// row per 16-key block).  The row's reference max m (scaled log2 units) enters the matrix
// core as the initial value of the Q.K^T accumulator, -m/c in raw score units, so the
// scores come back as S = s - m/c and the weights are 2^(c*S), c = sm_scale * log2(e) > 0.
// Per-row state kept per lane:
//   m    reference max (-inf before the row has seen an allowed key)
//   nm4  -m/c (0 while m is -inf) in four copies: the accumulator's initial value
//   l    this lane's share of the row sum of the weights, in units of 2^m
//   o    the output accumulator, in units of 2^m
// Exact step (a row's first key tile, and every tile that reaches the tree tail): the row
// max decides; a row that has no reference yet, or whose max exceeds the reference by more
// than kRebase, moves its reference to that max and rescales o and l.  Fast step (every
// other tile): the weights are formed against the current reference with no max at all,
// and only their per-lane sum is tested; a sum above kTripSum (or not finite) sends the
// tile back through the exact step before its weights are used.  Either way every weight
// is at most 2^64, so weights, row sums and outputs stay finite, and the final division by
// l cancels the reference: the result is exact up to rounding.

// Masked scores of the tree tail: `allow` holds this lane's allowed-key bits, bit 16*kb + i.
template <int KB>
__device__ inline void apply_mask(f32x4 (&sacc)[KB], uint64_t allow) {
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = 0; i < 4; ++i)
      sacc[kb][i] = ((allow >> (16 * kb + i)) & 1ull) ? sacc[kb][i] : -INFINITY;
}

// Exact step of one row tile (see above); moves S to the new reference in place.
template <int KB, int DB>
__device__ inline void rebase_exact(f32x4 (&sacc)[KB], float c, float& m, f32x4& nm4,
                                    float& l, f32x4 (&o)[DB]) {
  float mx = sacc[0][0];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int i = (kb == 0 ? 1 : 0); i < 4; ++i) mx = fmaxf(mx, sacc[kb][i]);
  mx = fmaxf(mx, __shfl_xor(mx, 16));
  mx = fmaxf(mx, __shfl_xor(mx, 32));  // row max of S, raw units
  const bool fresh = m == -INFINITY;
  const bool need = fresh ? mx != -INFINITY : mx * c > kRebase;
  if (__any(need)) {  // wave-uniform
    const float shift = need ? mx : 0.f;
    const float alpha = need ? (fresh ? 0.f : __builtin_amdgcn_exp2f(-mx * c)) : 1.f;
    l *= alpha;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db] *= alpha;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) sacc[kb] -= shift;
    nm4 -= shift;
    if (need) m = fresh ? mx * c : m + mx * c;
  }
}

// P = 2^(c*S) packed to bf16 as the B operand of P.V; returns this lane's sum of the same
// rounded values (dot with (1, 1)), so numerator and denominator use equal weights.
template <int KB, int KS>
__device__ inline float exp_pack(const f32x4 (&sacc)[KB], float c, bf16x8 (&pk)[KS]) {
  const bf16x2 ones = {static_cast<__bf16>(1.f), static_cast<__bf16>(1.f)};
  float lt = 0.f;
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const bf16x2 pair = {static_cast<__bf16>(__builtin_amdgcn_exp2f(sacc[kb][2 * h] * c)),
                           static_cast<__bf16>(__builtin_amdgcn_exp2f(sacc[kb][2 * h + 1] * c))};
      pk[kb >> 1][(kb & 1) * 4 + 2 * h] = pair[0];
      pk[kb >> 1][(kb & 1) * 4 + 2 * h + 1] = pair[1];
      lt = __builtin_amdgcn_fdot2_f32_bf16(pair, ones, lt, false);
    }
  return lt;
}

// Final store of one row: normalised output and natural-log LSE, or the split partial.
template <int D>
__device__ inline void store_row_block(const AttnParams& p, bool direct, int b, int hkv,
                                       int split, int node, int head, int row, int lh,
                                       const f32x4 (&o)[D / 16], float m, float lt) {
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  const float lse2 = lt > 0.f ? m + log2f(lt) : -INFINITY;
  if (direct) {
    uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)b * p.o_sb +
                    (int64_t)node * p.o_sn + (int64_t)head * p.o_sh;
#pragma unroll
    for (int db = 0; db < D / 16; ++db) {
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(o[db][i] * inv);
      *reinterpret_cast<bf16x4*>(out + db * 16 + 4 * lh) = v;
    }
    if (lh == 0 && p.lse) p.lse[((int64_t)b * p.N + node) * p.Hq + head] = lse2 * kLn2;
  } else {
    const int64_t prow = (((int64_t)b * p.Hkv + hkv) * p.num_splits + split) * p.R + row;
    float* dst = p.ws_o + prow * D;
#pragma unroll
    for (int db = 0; db < D / 16; ++db)
      *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * lh) = o[db] * inv;
    if (lh == 0) p.ws_lse[prow] = lse2;
  }
}

// Fused rotary embedding of the tree keys held by the window of tiles it .. it+WIN-1: every
// K row of logical key t in [L, kend) is rotated in place in LDS at position
// L + depth(t - L), from the workgroup's pair frequencies `inv_freq`; feature m of row r
// sits in chunk m/8 of the swizzled row, its partner
// m + D/2 in chunk m/8 + CH/2.  Called by every thread of the workgroup between the
// window's publishing barrier and a second barrier; V rows are untouched.  One pair per
// step and no unrolling, so the few registers it needs fit beside the loop's live state.
template <class C, int KT, int NST, int WIN>
__device__ inline void rope_tree_keys(char* smem, int it, int ntiles, int kbeg, int kend,
                                      int L, const uint64_t* mask_s, const double* inv_freq,
                                      int tid, int nthreads) {
  constexpr int H = C::CH * 4;  // pairs per row: half the row's features
  const int t_lo = max(L, kbeg + it * KT);
  const int t_hi = min(kend, kbeg + min(it + WIN, ntiles) * KT);
#pragma unroll 1
  for (int item = tid; item < (t_hi - t_lo) * H; item += nthreads) {
    const int t = t_lo + item / H;
    const int mm = item % H;
    const int tt = (t - kbeg) / KT;
    const int r = (t - kbeg) % KT;
    float cs, sn;
    rope_cos_sin_inv(L + depth_of(mask_s[t - L]), inv_freq[mm], cs, sn);
    char* row = smem + (tt % NST) * C::STAGEB + r * C::ROWB + (mm % 8) * 2;
    __bf16* px = reinterpret_cast<__bf16*>(row + (((mm / 8) ^ swz_k<C::CH>(r)) << 4));
    __bf16* py = reinterpret_cast<__bf16*>(row + (((mm / 8 + C::CH / 2) ^ swz_k<C::CH>(r)) << 4));
    float x = static_cast<float>(*px), y = static_cast<float>(*py);
    rope_pair(x, y, cs, sn);
    *px = static_cast<__bf16>(x);
    *py = static_cast<__bf16>(y);
  }
}

// The same, called out of line: shapes that keep the shared remainder tile hold ~250
// registers through the loop, and the rotation's fp64 temporaries would otherwise spill
// loop state.  A spill reload inside the loop waits on the vector-memory counter, which
// also counts the ring's direct loads, so every reload would drain the ring.
template <class C, int KT, int NST, int WIN>
__device__ __noinline__ void rope_tree_keys_outlined(char* smem, int it, int ntiles, int kbeg,
                                                     int kend, int L, const uint64_t* mask_s,
                                                     const double* inv_freq, int tid,
                                                     int nthreads) {
  rope_tree_keys<C, KT, NST, WIN>(smem, it, ntiles, kbeg, kend, L, mask_s, inv_freq, tid,
                                  nthreads);
}

// Fused rotary embedding of one wave's Q operand registers of one tile: the lane parks its
// DS operands in a private LDS slot, rotates them there with a plain loop (register arrays
// take static indices only) by the cos/sin of its node's row `cs_row` (one per feature
// pair) and reloads them.  Feature
// m = 32s + 8lh + e sits in operand s, element e; its partner m + D/2 in operand s + DS/2.
template <int D>
__device__ inline void rope_q_tile(bf16x8 (&q)[D / 32], char* slot, const float2* cs_row,
                                   int lh) {
  constexpr int DS = D / 32;
#pragma unroll
  for (int s = 0; s < DS; ++s) *reinterpret_cast<bf16x8*>(slot + 16 * 64 * s) = q[s];
#pragma unroll 1
  for (int i = 0; i < DS / 2 * 8; ++i) {
    const int s = i / 8, e = i % 8;
    const float2 t = cs_row[32 * s + 8 * lh + e];
    const float cs = t.x, sn = t.y;
    __bf16* px = reinterpret_cast<__bf16*>(slot + 16 * 64 * s) + e;
    __bf16* py = reinterpret_cast<__bf16*>(slot + 16 * 64 * (s + DS / 2)) + e;
    float x = static_cast<float>(*px), y = static_cast<float>(*py);
    rope_pair(x, y, cs, sn);
    *px = static_cast<__bf16>(x);
    *py = static_cast<__bf16>(y);
  }
#pragma unroll
  for (int s = 0; s < DS; ++s) q[s] = *reinterpret_cast<const bf16x8*>(slot + 16 * 64 * s);
}

// TN full 16-node tiles per wave (wave w = query head w of the group).  RR = 1 adds the
// shared remainder tile: the N - 16*TN nodes past the full tiles, packed node-major
// across the g heads (row = (node - 16*TN) * g + head), computed by wave it % NW on key
// tile `it`; each wave keeps its own online-softmax partial of that tile and the partials
// are merged through LDS at the end (the same maths as the split merge).
// TEAMS = 2 (grids of at most one workgroup per compute unit): two teams of NW waves, so
// each SIMD holds a wave of each; every window of 2 * TEAMS key tiles gives each team two
// of them, and at the end team 1's online-softmax partials merge into team 0's through
// LDS.  One prologue and one partial per workgroup, as with one team.
template <int D, int KT, int NST, int TN, int RR, int NW, bool ROPE, int TEAMS, bool PG>
__global__ void __launch_bounds__(NW * 64 * TEAMS, TEAMS == 1 ? 2 : 1)
    tv_attn_mfma_kernel(AttnParams p) {
  using C = MfmaCfg<D, KT, NST, TN, NW>;
  constexpr int DS = C::DS, DB = C::DB, KB = C::KB, KS = C::KS;
  constexpr int TT = TN + RR;  // tiles of state per wave: full tiles, then the shared one
  constexpr int NTH = NW * 64 * TEAMS;  // threads of the workgroup
  static_assert(TEAMS == 1 || (TEAMS == 2 && !ROPE), "teams: the plain pass only");
  __shared__ __attribute__((aligned(1024))) char smem[NST * C::STAGEB];
  __shared__ uint64_t mask_s[TV_MAX_NODES];
  __shared__ int32_t par_s[TV_MAX_NODES];
  __shared__ int32_t pt_s[kMaxPageSlice];
  // the shared remainder tile's query operands (B-operand layout, [k-step][lane]): read
  // from LDS on the key tiles a wave computes it, so they take no registers in the loop
  __shared__ bf16x8 qrem_s[RR ? DS * 64 : 1];
  // rotary pair frequencies, formed once in fp64 (fused RoPE only)
  __shared__ double inv_s[ROPE ? D / 2 : 1];
  static_assert(!RR || TEAMS * NW * 16 * D * 4 <= NST * C::STAGEB, "merge buffer fits the ring");
  static_assert(!RR || TEAMS * NW * 16 * 2 <= kMaxPageSlice, "merge (m, l) fits the page slice");
  static_assert(TEAMS == 1 || NW * TN * DB * 64 * 16 + NW * TN * 64 * 8 <= NST * C::STAGEB,
                "team merge buffer fits the ring");

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave of the workgroup
  const int team = TEAMS == 1 ? 0 : wv / NW;                // 0 unless TEAMS == 2
  const int w = TEAMS == 1 ? wv : wv - team * NW;           // wave within its team
  const int lr = lane & 15;
  const int lh = lane >> 4;
  const int hkv = blockIdx.y % p.Hkv;
  const int hc = (blockIdx.y / p.Hkv) % p.head_chunks;
  const int t0 = (blockIdx.y / p.Hkv / p.head_chunks) * TN;  // first 16-node tile of this wg
  static_assert(3 * kMaxLptBatch + 1 <= kMaxPageSlice, "piece order fits the page slice");
  int b = blockIdx.z, split = blockIdx.x;
  if (p.lpt) {
    if (!lpt_piece(p, blockIdx.z * gridDim.x + blockIdx.x, pt_s, tid, NTH, b, split))
      return;  // more slots than pieces
    b = __builtin_amdgcn_readfirstlane(b);
    split = __builtin_amdgcn_readfirstlane(split);
  }
  const int L = clamped_prefix(p, b);
  const int Ttot = L + p.N;
  const bool direct = single_split(p, Ttot);  // no merge for this request
  const int kbeg = split * p.chunk;
  if (kbeg >= Ttot) return;  // this request has fewer splits than the grid
  const int kend = min(kbeg + p.chunk, Ttot);
  const int ntiles = (kend - kbeg + KT - 1) / KT;

  const char* kg = static_cast<const char*>(p.k);
  const char* vg = static_cast<const char*>(p.v);
  const uint32_t sbase = (uint32_t)(uintptr_t)(TV_LDS char*)smem;

  // Two-team shapes (grids of at most one workgroup per compute unit) over contiguous KV:
  // this team's full tiles of the first window go out before the prologue's own loads, so
  // that their latency overlaps the query loads and the ancestor walk; the prologue's final
  // wait drains them with its own loads.  The ring is idle until the key loop (fused RoPE
  // uses it as scratch, so it keeps the order below).  Larger grids keep that order too:
  // there every workgroup's early tiles only queue behind the others' (1-3% slower).
  constexpr bool EARLY = TEAMS == 2 && !ROPE && !PG;
  if constexpr (EARLY) {
    if (!p.paged && (int64_t)(KT - 1) * p.kv_st * 2 + 2 * D <= INT32_MAX) {
      const LoadPlan<C, NW> lpe(p, w, lane);
      RowMap rme;
      rme.pt = pt_s;
      rme.pbase = 0;
      rme.head_off = (int64_t)b * p.kv_sb + (int64_t)hkv * p.kv_sh;
#pragma unroll
      for (int s = 0; s < 2 * TEAMS; ++s)  // window 0: two tiles per team
        if (s / 2 == team && s < ntiles && kbeg + (s + 1) * KT <= kend)
          issue_tile<C, NW, KT, false>(p, rme, lpe, kg, vg, sbase + s * C::STAGEB, kbeg + s * KT,
                                       kend, true, false, w, lane);
    }
  }

  // ---- prologue: every compiler-visible global load (Q, parent array, page-table slice)
  // happens here and is drained by one explicit wait before the asm-issued ring starts;
  // otherwise the compiler would guard later uses of these registers with vmcnt(0) and
  // drain the ring on every tile.
  const int j = hc * NW + w;              // query head within the kv head's group
  const bool head_on = j < p.g;           // wave-uniform
  const int head = hkv * p.g + (head_on ? j : 0);
  const int rem_rows = RR ? (p.N - 16 * TN) * p.g : 0;  // valid rows of the shared tile
  bf16x8 qreg[TT][DS];
  int node_of[TT];  // tree node of this lane's row in each tile, clamped into [0, N)
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    int node, hd;
    bool valid;
    if (t < TN) {  // full tiles: head-major (rows past N are padding)
      node = (t0 + t) * 16 + lr;
      hd = head;
      valid = head_on && node < p.N;
    } else {       // shared remainder tile: node-major across the group's heads
      node = 16 * TN + lr / p.g;
      hd = hkv * p.g + lr % p.g;
      valid = head_on && lr < rem_rows;
    }
    node_of[t] = min(node, p.N - 1);
    const uint16_t* src = static_cast<const uint16_t*>(p.q) + (int64_t)b * p.q_sb +
                          (int64_t)(valid ? node : 0) * p.q_sn +
                          (int64_t)(valid ? hd : 0) * p.q_sh + 8 * lh;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (valid) v = *reinterpret_cast<const uint4*>(src + 32 * s);
      qreg[t][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  // The parent array is staged in LDS with one coalesced load, so that each node's walk up
  // to the root chases its parent links through LDS rather than through global memory (a
  // round trip per level, all before the key ring may start).
  if (tid < p.N) par_s[tid] = p.parent[(int64_t)b * p.parent_sb + tid];
  __syncthreads();
  if (tid < p.N) {
    bool ok;
    int dd;
    const uint64_t m = ancestor_bits(par_s, tid, p.N, ok, dd);
    mask_s[tid] = m;
    // one workgroup per request (split 0, first row chunk of kv head 0) exports the tree
    if (split == 0 && blockIdx.y == 0) export_node_meta(p, b, tid, m, ok, dd);
  }

  RowMap rm;
  rm.pt = pt_s;
  rm.pbase = 0;
  if (p.paged) {
    // this split's slice of the page table, staged once in LDS (the host bounds its size)
    rm.head_off = (int64_t)hkv * p.kv_sh;
    rm.pbase = p.page_shift >= 0 ? (kbeg >> p.page_shift) : kbeg / p.page_size;
    const int plast = p.page_shift >= 0 ? ((kend - 1) >> p.page_shift) : (kend - 1) / p.page_size;
    const int32_t* prow = p.page_table + (int64_t)b * p.pages_per_seq;
    for (int i = tid; i <= plast - rm.pbase; i += NTH) pt_s[i] = prow[rm.pbase + i];
  } else {
    rm.head_off = (int64_t)b * p.kv_sb + (int64_t)hkv * p.kv_sh;
  }
  wait_vmcnt<0>();
  __syncthreads();  // mask_s and pt_s visible

  if constexpr (ROPE) {
    // ---- fused rotary embedding of the queries, node i at L + depth(i), in lane-private
    // LDS slots of the (still idle) ring: DS KB per wave.  The cos/sin of every (node of
    // this workgroup's tiles, feature pair) are formed once per workgroup into a table
    // after the slots (the waves' query heads share positions), from the pair frequencies
    // formed once in fp64. ----
    constexpr int H = D / 2;
    static_assert(NW * DS * 1024 + TT * 16 * H * 8 <= NST * C::STAGEB,
                  "query slots and the cos/sin table fit the ring");
    const int nbase = t0 * 16;                         // first node of this workgroup's tiles
    const int nrows = min(p.N - nbase, TT * 16);       // node_of[t] - nbase < nrows
    float2* cs_tab = reinterpret_cast<float2*>(smem + NW * DS * 1024);
    if (tid < H) inv_s[tid] = rope_inv_freq(tid, D, p.rope_log2_theta);
    __syncthreads();
    for (int idx = tid; idx < nrows * H; idx += NTH) {
      const int i = idx / H, m = idx - (idx / H) * H;
      float cs, sn;
      rope_cos_sin_inv(L + depth_of(mask_s[nbase + i]), inv_s[m], cs, sn);
      cs_tab[idx] = make_float2(cs, sn);
    }
    __syncthreads();
    char* slot = smem + w * DS * 1024 + 16 * lane;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      // only wave 0 parks the shared remainder tile's queries; the others drop theirs
      if (t >= TN && w != 0) continue;
      rope_q_tile<D>(qreg[t], slot, cs_tab + (node_of[t] - nbase) * H, lh);
    }
    __syncthreads();  // the ring may now be overwritten
  }

  // ---- park the remainder tile's query operands in LDS ----
  const float c = p.scale_log2;
  if constexpr (RR) {
    if (wv == 0) {
#pragma unroll
      for (int s = 0; s < DS; ++s) qrem_s[s * 64 + lane] = qreg[TN][s];
    }
    __syncthreads();  // qrem_s visible before the first remainder tile
  }

  // ---- start the first two windows streaming (each team loads its own tiles) ----
  constexpr int WIN = 2;           // tiles a team computes per window
  constexpr int SW = WIN * TEAMS;  // tiles per window of the workgroup
  static_assert(NST == 2 * SW, "a ring of two windows");
  const LoadPlan<C, NW> lp(p, w, lane);
  const bool off32 = (int64_t)(KT - 1) * p.kv_st * 2 + 2 * D <= INT32_MAX;
  // the paged instantiation compiles the contiguous path out (the launcher sends it paged
  // calls only); the contiguous one keeps the run-time test, as does its prologue.  The
  // vector form of the paged addresses holds two more registers across the load issue:
  // the two-team shapes and three-tile waves with fused RoPE have none to spare (they
  // would spill inside the loop), so they keep the scalar form.
  constexpr bool VA = PG && TEAMS == 1 && !(ROPE && TN >= 3);
  const bool fast = !PG && !p.paged && off32;
  const bool pfast = p.paged && off32 && p.page_shift >= 0 && p.page_size % C::RPI == 0;
  static_assert(!EARLY || WIN == 2, "the early issue assumes two-tile windows");
#pragma unroll
  for (int s = 0; s < NST; ++s)
    if (s < ntiles && (s / WIN) % TEAMS == team &&
        !(EARLY && fast && s < SW && kbeg + (s + 1) * KT <= kend))  // not issued early
      issue_tile<C, NW, KT, VA>(p, rm, lp, kg, vg, sbase + s * C::STAGEB, kbeg + s * KT, kend,
                                fast, pfast, w, lane);

  f32x4 o[TT][DB];
  f32x4 nm4[TT];
  float m[TT], l[TT];
#pragma unroll
  for (int t = 0; t < TT; ++t) {
    m[t] = -INFINITY;
    nm4[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    l[t] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // One key tile: S^T = K Q^T, mask, online softmax, O^T += V^T P^T.  `it` is the tile's
  // index in the split, `k` its index among the tiles this wave's team computes (the same
  // with one team): a row tile's first tile, k == 0, and the remainder tile's first
  // (k < NW) take the exact step.
  auto tile = [&](int it, int k, bool do_rem, auto young_c) {
    constexpr bool young = decltype(young_c)::value;
    const int kt0 = kbeg + it * KT;
    const char* ks = smem + (it % NST) * C::STAGEB;
    const char* vs = ks + C::TILEB;

    // ---- S^T = K Q^T (raised issue priority: see mfma_priority) ----
    mfma_priority(true, young);
    bf16x8 qr[DS];
    if (RR && do_rem) {
#pragma unroll
      for (int s = 0; s < DS; ++s) qr[s] = qrem_s[s * 64 + lane];
    }
    f32x4 sacc[TT][KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = kb * 16 + lr;
      bf16x8 ka[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s)
        ka[s] = *reinterpret_cast<const bf16x8*>(ks + r * C::ROWB +
                                                 (((4 * s + lh) ^ swz_k<C::CH>(r)) << 4));
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t >= TN && !do_rem) continue;
        f32x4 acc = nm4[t];  // scores come back relative to the row's reference
#pragma unroll
        for (int s = 0; s < DS; ++s)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], t < TN ? qreg[t][s] : qr[s], acc,
                                                        0, 0, 0);
        sacc[t][kb] = acc;
      }
    }

    mfma_priority(false, young);
    // ---- weights: exact step on a row tile's first key tile and on the tree tail, fast
    // step with the row-sum test elsewhere ----
    const bool masked = kt0 + KT > L;
    bf16x8 pk[TT][KS];
    float lt[TT];
    bool trip = false;
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= TN && !do_rem) continue;
      // a full tile's first key tile is the split's first; the remainder tile's is the
      // first this wave computes (it < NW)
      const bool exact = masked || (t < TN ? k == 0 : k < NW);
      if (exact) {
        if (masked) apply_mask<KB>(sacc[t], tile_allowed(mask_s[node_of[t]], kt0, L) >> (4 * lh));
        rebase_exact<KB, DB>(sacc[t], c, m[t], nm4[t], l[t], o[t]);
      }
      lt[t] = exp_pack<KB, KS>(sacc[t], c, pk[t]);
      if (!exact) trip |= !(lt[t] <= kTripSum);
    }
    if (__any(trip)) {  // wave-uniform; never on ordinary data after a row's first tile
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t >= TN && !do_rem) continue;
        if (masked || (t < TN ? k == 0 : k < NW)) continue;
        if (__any(!(lt[t] <= kTripSum))) {
          rebase_exact<KB, DB>(sacc[t], c, m[t], nm4[t], l[t], o[t]);
          lt[t] = exp_pack<KB, KS>(sacc[t], c, pk[t]);
        }
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      if (t >= TN && !do_rem) continue;
      l[t] += lt[t];
    }

    // ---- O^T += V^T P^T, V^T read transposed from V's row-major tile.  The operand of
    // feature block db+1 is read before the MFMAs of block db, so the LDS latency of every
    // block but the first overlaps matrix work. ----
    const int q4 = lr & 3;                       // which 4-feature group this lane addresses
    auto read_v = [&](int db, int kss) {
      const int chunk = 2 * db + (q4 >> 1);      // 16-byte chunk of features 16db + 4q4
      const int half = (q4 & 1) << 3;            // byte offset inside the chunk
      const int r0 = 32 * kss + 4 * lh + (lr >> 2);
      const int r1 = r0 + 16;
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (TV_LDS v4i16*)(vs + r0 * C::ROWB + ((chunk ^ swz_v<C::CH>(r0)) << 4) + half));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (TV_LDS v4i16*)(vs + r1 * C::ROWB + ((chunk ^ swz_v<C::CH>(r1)) << 4) + half));
      return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    };
    mfma_priority(true, young);
    constexpr int NV = DB * KS;                  // V operands per tile, db-major
    constexpr int PF = 1;                        // operands in flight ahead of the MFMAs
    bf16x8 va[PF + 1];
#pragma unroll
    for (int iv = 0; iv < PF && iv < NV; ++iv) va[iv] = read_v(iv / KS, iv % KS);
#pragma unroll
    for (int iv = 0; iv < NV; ++iv) {
      const int db = iv / KS, kss = iv % KS;
      if (iv + PF < NV) va[(iv + PF) % (PF + 1)] = read_v((iv + PF) / KS, (iv + PF) % KS);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        if (t >= TN && !do_rem) continue;
        o[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[iv % (PF + 1)], pk[t][kss],
                                                           o[t][db], 0, 0, 0);
      }
    }
    mfma_priority(false, young);
  };

  // Tiles go in windows of SW = TEAMS * WIN: one barrier per window publishes its tiles and
  // frees the stages of the previous window, whose loads for the next window then stream
  // while this one is computed; team t computes (and loads) tiles t*WIN .. t*WIN+WIN-1 of
  // every window.  The shared remainder tile of a key tile is computed by wave k % NW of
  // the team that has the tile, k the tile's index among that team's tiles, so within a
  // window the extra work lands on WIN different waves of each team.
  // The loop is compiled twice, for the older and the younger workgroup of a unit, so the
  // priority switches inside the tiles take no branch.
  auto key_loop = [&](auto young_c) {
    const int own = team * WIN;  // this team's first tile within a window
    for (int it = 0; it < ntiles; it += SW) {
      if (it == 0) {
        // the prologue issued this team's tiles of windows 0 and 1; those of window 1 may
        // remain in flight
        if constexpr (TEAMS == 1)
          wait_tiles<C::LPW, WIN>(min(ntiles, NST) - min(ntiles, WIN));
        else
          wait_tiles<C::LPW, WIN>(max(0, min(ntiles - SW - own, WIN)));
      } else {
        wait_vmcnt<0>();  // this window's tiles were the last ones this wave issued
      }
      __syncthreads();  // window visible to all waves; the previous window's stages are free
      if (it > 0) {
#pragma unroll
        for (int s = 0; s < WIN; ++s) {
          const int tn = it + SW + own + s;
          if (tn < ntiles)
            issue_tile<C, NW, KT, VA>(p, rm, lp, kg, vg, sbase + (tn % NST) * C::STAGEB,
                                      kbeg + tn * KT, kend, fast, pfast, w, lane);
        }
      }
      if (ROPE && kbeg + (it + WIN) * KT > L) {  // the window holds tree keys (uniform)
        if constexpr (RR)
          rope_tree_keys_outlined<C, KT, NST, WIN>(smem, it, ntiles, kbeg, kend, L, mask_s,
                                                   inv_s, tid, NW * 64);
        else
          rope_tree_keys<C, KT, NST, WIN>(smem, it, ntiles, kbeg, kend, L, mask_s, inv_s, tid,
                                          NW * 64);
        __syncthreads();
      }
      if (!head_on) continue;  // surplus wave of a group smaller than NW: loads only
#pragma unroll
      for (int s = 0; s < WIN; ++s) {
        const int tt = it + own + s;
        const int k = TEAMS == 1 ? tt : it / TEAMS + s;  // this team's tile count so far
        if (tt < ntiles) tile(tt, k, RR && (k % NW) == w, young_c);
      }
    }
  };
  // the shapes the host may flag (three-tile waves would spill with two copies of the loop)
  if constexpr (NW == 4 && TN <= 2 && TEAMS == 1) {
    if ((int)((blockIdx.z * gridDim.y + blockIdx.y) * gridDim.x + blockIdx.x) >= p.young_from)
      key_loop(std::true_type{});
    else
      key_loop(std::false_type{});
  } else {
    key_loop(std::false_type{});
  }

  if constexpr (TEAMS == 2) {
    // ---- team 1's partials of the full tiles merge into team 0's through LDS ----
    f32x4* xo = reinterpret_cast<f32x4*>(smem);                        // [NW][TN][DB][64]
    float* xm = reinterpret_cast<float*>(smem + NW * TN * DB * 64 * 16);  // [NW][TN][64] x (m, l)
    __syncthreads();  // every wave is done with the ring
    if (team == 1 && head_on) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
#pragma unroll
        for (int db = 0; db < DB; ++db) xo[((w * TN + t) * DB + db) * 64 + lane] = o[t][db];
        xm[((w * TN + t) * 64 + lane) * 2] = m[t];
        xm[((w * TN + t) * 64 + lane) * 2 + 1] = l[t];
      }
    }
    __syncthreads();
    if (team == 0 && head_on) {
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const float m1 = xm[((w * TN + t) * 64 + lane) * 2];
        const float l1 = xm[((w * TN + t) * 64 + lane) * 2 + 1];
        const float mx = fmaxf(m[t], m1);
        const float s0 = m[t] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m[t] - mx);
        const float s1 = m1 == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m1 - mx);
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[t][db] = o[t][db] * s0 + xo[((w * TN + t) * DB + db) * 64 + lane] * s1;
        l[t] = l[t] * s0 + l1 * s1;
        m[t] = mx;
      }
    }
  }

  // ---- epilogue: full tiles straight from registers ----
  if (head_on && team == 0) {
#pragma unroll
    for (int t = 0; t < TN; ++t) {
      float lt = l[t];
      lt += __shfl_xor(lt, 16);
      lt += __shfl_xor(lt, 32);
      const int node = (t0 + t) * 16 + lr;
      if (node < p.N)
        store_row_block<D>(p, direct, b, hkv, split, node, head, node * p.g + j, lh, o[t],
                           m[t], lt);
    }
  }
  if constexpr (RR) {
    // ---- shared remainder tile: merge the waves' partials through LDS ----
    float* mo = reinterpret_cast<float*>(smem);   // [TEAMS * NW][16][D] unnormalised O
    float* ml = reinterpret_cast<float*>(pt_s);   // [TEAMS * NW][16] x (m, l)
    __syncthreads();                              // every wave is done with the ring
    float lt = l[TN];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
#pragma unroll
    for (int db = 0; db < DB; ++db)
      *reinterpret_cast<f32x4*>(mo + (wv * 16 + lr) * D + db * 16 + 4 * lh) = o[TN][db];
    if (lh == 0) {
      ml[(wv * 16 + lr) * 2] = head_on ? m[TN] : -INFINITY;
      ml[(wv * 16 + lr) * 2 + 1] = head_on ? lt : 0.f;
    }
    __syncthreads();
    for (int item = tid; item < 16 * (D / 4); item += NTH) {
      const int row = item / (D / 4);
      const int q4 = item % (D / 4);
      if (row >= rem_rows) continue;
      float M = -INFINITY;
#pragma unroll
      for (int ww = 0; ww < TEAMS * NW; ++ww) M = fmaxf(M, ml[(ww * 16 + row) * 2]);
      float Ls = 0.f;
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
      if (M != -INFINITY) {
#pragma unroll
        for (int ww = 0; ww < TEAMS * NW; ++ww) {
          const float mw = ml[(ww * 16 + row) * 2];
          if (mw == -INFINITY) continue;
          const float sc = __builtin_amdgcn_exp2f(mw - M);
          Ls += sc * ml[(ww * 16 + row) * 2 + 1];
          acc += sc * *reinterpret_cast<const f32x4*>(mo + (ww * 16 + row) * D + 4 * q4);
        }
      }
      const int node = 16 * TN + row / p.g;
      const int hd = hkv * p.g + row % p.g;
      const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
      const float lse2 = Ls > 0.f ? M + log2f(Ls) : -INFINITY;
      if (direct) {
        uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)b * p.o_sb +
                        (int64_t)node * p.o_sn + (int64_t)hd * p.o_sh + 4 * q4;
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(acc[i] * inv);
        *reinterpret_cast<bf16x4*>(out) = v;
        if (q4 == 0 && p.lse) p.lse[((int64_t)b * p.N + node) * p.Hq + hd] = lse2 * kLn2;
      } else {
        const int64_t prow =
            (((int64_t)b * p.Hkv + hkv) * p.num_splits + split) * p.R + node * p.g + row % p.g;
        *reinterpret_cast<f32x4*>(p.ws_o + prow * D + 4 * q4) = acc * inv;
        if (q4 == 0) p.ws_lse[prow] = lse2;
      }
    }
  }
}

constexpr int kMfmaKT = 32;
constexpr int kMfmaNST = 4;

template <int D, bool ROPE, int TEAMS, bool PG>
static hipError_t launch_d(const AttnParams& p, MfmaShape sh, hipStream_t s) {
  dim3 grid(p.num_splits, p.Hkv * p.row_chunks, p.B);
#define TV_CASE(TN, RR, NW)                                                                  \
  if (sh.tpw == TN && sh.rr == RR && sh.nw == NW) {                                          \
    hipLaunchKernelGGL(                                                                      \
        (tv_attn_mfma_kernel<D, kMfmaKT, kMfmaNST * TEAMS, TN, RR, NW, ROPE, TEAMS, PG>),    \
        grid,                                                                                \
        dim3(NW * 64 * TEAMS), 0, s, p);                                                     \
    return hipGetLastError();                                                                \
  }
  if constexpr (TEAMS == 2) {  // four-wave groups only (the host flags no others)
    TV_CASE(1, 0, 4) TV_CASE(2, 0, 4) TV_CASE(3, 0, 4) TV_CASE(1, 1, 4) TV_CASE(2, 1, 4)
    return hipErrorInvalidConfiguration;
  } else {
    TV_CASE(1, 0, 1) TV_CASE(1, 0, 2) TV_CASE(1, 0, 4) TV_CASE(1, 0, 8)
    TV_CASE(2, 0, 1) TV_CASE(2, 0, 2) TV_CASE(2, 0, 4) TV_CASE(2, 0, 8)
    TV_CASE(3, 0, 1) TV_CASE(3, 0, 2) TV_CASE(3, 0, 4) TV_CASE(3, 0, 8)
    TV_CASE(1, 1, 2) TV_CASE(1, 1, 4) TV_CASE(1, 1, 8)
    TV_CASE(2, 1, 2) TV_CASE(2, 1, 4) TV_CASE(2, 1, 8)
  }
#undef TV_CASE
  return hipErrorInvalidConfiguration;
}

// Every shape of one KV layout (PG: paged).
template <bool PG>
hipError_t launch_attn_mfma_layout(const AttnParams& p, int D, MfmaShape shape, hipStream_t s) {
  if (p.rope)
    return D == 64 ? launch_d<64, true, 1, PG>(p, shape, s)
                   : launch_d<128, true, 1, PG>(p, shape, s);
  if (D == 128 && shape.teams == 2) return launch_d<128, false, 2, PG>(p, shape, s);
  return D == 64 ? launch_d<64, false, 1, PG>(p, shape, s)
                 : launch_d<128, false, 1, PG>(p, shape, s);
}

}  // namespace tv
