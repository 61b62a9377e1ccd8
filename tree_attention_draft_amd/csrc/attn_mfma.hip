// Tree-verify attention, MFMA path (bf16 inputs, fp32 accumulation, gfx950).
//
// Semantics ("Tree attention mask for draft-tree verification", "A strong answer";
// "Tree Verification", "Tree Attention"): packed row r = node * g + j (g = Hq/Hkv) is query
// head hkv*g + j of tree node r / g; it attends every prefix key t < L and tree key L + i
// exactly when bit i of the node's ancestor bitmask is set.  The bitmask is built in LDS
// from the parent array once per workgroup and expanded per key tile; prefix tiles carry
// no mask at all.
//
// Work decomposition.  One workgroup = (key split, kv head [x row chunk], request).  All
// N*g query rows of the kv head are packed node-major and cut into 16-row tiles; wave w
// owns TPW consecutive tiles.  Each 64-key tile of K and V is read from HBM once per
// workgroup, staged in LDS, and reused by every wave, i.e. by all heads and nodes of the
// group.
//
// Matrix-core layout (v_mfma_f32_16x16x32_bf16; lane l, lr = l % 16, lh = l / 16):
//   A operand: row lr, k = 8*lh .. 8*lh+7;  B operand: column lr, same k;
//   result:    rows 4*lh .. 4*lh+3 of column lr.
// Scores are computed transposed, S^T = K Q^T (A = K tile from LDS, B = Q from registers),
// so every lane holds 4 keys of ONE query row: the row max / sum are in-lane plus two
// cross-lane steps.  The output is accumulated transposed too, O^T += V^T P^T: the P
// values a lane owns (keys 4lh..4lh+3 of two 16-key blocks) are exactly a B operand once
// the contraction index is permuted consistently, so P never leaves registers; V is
// stored transposed in LDS so the matching A operand is two 8-byte reads.
#include "kernels_common.h"

namespace tv {

template <int D, int TPW, int NW>
__global__ void __launch_bounds__(NW * 64) tv_attn_mfma_kernel(AttnParams p) {
  constexpr int KT = kKeysPerTile;  // 64
  constexpr int NT = NW * 64;
  constexpr int DS = D / 32;        // k-steps of Q.K^T
  constexpr int DB = D / 16;        // 16-feature output blocks
  constexpr int KPAD = D + 8;       // K row pitch in elements (+16 B against bank conflicts)
  constexpr int VPAD = KT + 4;      // V^T row pitch in elements (+8 B)
  constexpr int KCH = D / 8;        // 16-byte chunks per key row
  __shared__ __attribute__((aligned(16))) __bf16 Ks[KT * KPAD];
  __shared__ __attribute__((aligned(16))) __bf16 Vt[D * VPAD];
  __shared__ uint64_t mask_s[TV_MAX_NODES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int lr = lane & 15;
  const int lh = lane >> 4;
  const int split = blockIdx.x;
  const int hkv = blockIdx.y % p.Hkv;
  const int rc = blockIdx.y / p.Hkv;
  const int b = blockIdx.z;
  const int L = clamped_prefix(p, b);
  const int Ttot = L + p.N;
  const int kbeg = split * p.chunk;
  if (kbeg >= Ttot) return;  // this request has fewer splits than the grid
  const int kend = min(kbeg + p.chunk, Ttot);

  const uint16_t* __restrict__ qg = static_cast<const uint16_t*>(p.q);
  const uint16_t* __restrict__ kg = static_cast<const uint16_t*>(p.k);
  const uint16_t* __restrict__ vg = static_cast<const uint16_t*>(p.v);

  if (tid < p.N) {
    bool ok;
    int dd;
    mask_s[tid] = ancestor_bits(p.parent + (int64_t)b * p.parent_sb, tid, p.N, ok, dd);
  }

  // ---- this wave's query tiles, as B operands (column = packed row, k = feature) ----
  const int qt0 = (rc * NW + w) * TPW;  // first 16-row tile of this wave
  bf16x8 qreg[TPW][DS];
  int row_node[TPW];
  bool tile_on[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int row = (qt0 + t) * 16 + lr;
    tile_on[t] = (qt0 + t) * 16 < p.R;  // wave-uniform
    const bool valid = row < p.R;
    const int node = valid ? row / p.g : 0;
    const int head = hkv * p.g + (valid ? row % p.g : 0);
    row_node[t] = node;
    const uint16_t* src = qg + (int64_t)b * p.q_sb + (int64_t)node * p.q_sn +
                          (int64_t)head * p.q_sh + 8 * lh;
#pragma unroll
    for (int s = 0; s < DS; ++s) {
      uint4 v = make_uint4(0, 0, 0, 0);
      if (valid) v = *reinterpret_cast<const uint4*>(src + 32 * s);
      qreg[t][s] = __builtin_bit_cast(bf16x8, v);
    }
  }

  f32x4 o[TPW][DB];
  float m[TPW], l[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[t][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();  // mask_s ready
  uint64_t rmask[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) rmask[t] = mask_s[row_node[t]];

  const float c = p.scale_log2;

  for (int kt0 = kbeg; kt0 < kend; kt0 += KT) {
    // ---- stage K (row-major) and V (transposed) for keys [kt0, kt0 + 64) in LDS ----
    for (int ci = tid; ci < KT * KCH; ci += NT) {
      const int key = ci / KCH, ch = ci - (ci / KCH) * KCH;
      const int t = kt0 + key;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (t < kend) v = *reinterpret_cast<const uint4*>(kg + kv_offset(p, b, t, hkv) + 8 * ch);
      *reinterpret_cast<uint4*>(&Ks[key * KPAD + 8 * ch]) = v;
    }
    for (int ui = tid; ui < (KT / 4) * KCH; ui += NT) {
      const int kq = ui / KCH, ch = ui - (ui / KCH) * KCH;
      uint4 r[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = kt0 + 4 * kq + e;
        r[e] = make_uint4(0, 0, 0, 0);
        if (t < kend) r[e] = *reinterpret_cast<const uint4*>(vg + kv_offset(p, b, t, hkv) + 8 * ch);
      }
      const uint32_t* w0 = reinterpret_cast<const uint32_t*>(&r[0]);
      const uint32_t* w1 = reinterpret_cast<const uint32_t*>(&r[1]);
      const uint32_t* w2 = reinterpret_cast<const uint32_t*>(&r[2]);
      const uint32_t* w3 = reinterpret_cast<const uint32_t*>(&r[3]);
#pragma unroll
      for (int wi = 0; wi < 4; ++wi) {
        uint2 even, odd;  // features 2*wi and 2*wi+1 of the four keys
        even.x = (w0[wi] & 0xFFFFu) | (w1[wi] << 16);
        even.y = (w2[wi] & 0xFFFFu) | (w3[wi] << 16);
        odd.x = (w0[wi] >> 16) | (w1[wi] & 0xFFFF0000u);
        odd.y = (w2[wi] >> 16) | (w3[wi] & 0xFFFF0000u);
        const int d0 = 8 * ch + 2 * wi;
        *reinterpret_cast<uint2*>(&Vt[d0 * VPAD + 4 * kq]) = even;
        *reinterpret_cast<uint2*>(&Vt[(d0 + 1) * VPAD + 4 * kq]) = odd;
      }
    }
    __syncthreads();

    // ---- S^T = K Q^T for this wave's tiles ----
    f32x4 sacc[TPW][4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      bf16x8 ka[DS];
#pragma unroll
      for (int s = 0; s < DS; ++s)
        ka[s] = *reinterpret_cast<const bf16x8*>(&Ks[(kb * 16 + lr) * KPAD + 32 * s + 8 * lh]);
#pragma unroll
      for (int t = 0; t < TPW; ++t) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
        if (tile_on[t]) {
#pragma unroll
          for (int s = 0; s < DS; ++s)
            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[s], qreg[t][s], acc, 0, 0, 0);
        }
        sacc[t][kb] = acc;
      }
    }

    // ---- mask (tree tail only), online softmax, P packing ----
    // Lane (lr, lh) holds keys kt0 + 16*kb + 4*lh + i of its row: bit 16*kb + i of the
    // tile's allowed word shifted down by 4*lh.
    const bool masked = kt0 + KT > L;
    bf16x8 pk[TPW][2];
#pragma unroll
    for (int t = 0; t < TPW; ++t) {
      if (masked) {
        const uint64_t allow = tile_allowed(rmask[t], kt0, L) >> (4 * lh);
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            sacc[t][kb][i] = ((allow >> (16 * kb + i)) & 1ull) ? sacc[t][kb][i] : -INFINITY;
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sacc[t][kb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16));
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float m_new = fmaxf(m[t], mx * c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m[t] - m_use);
      m[t] = m_new;
      float rs = 0.f;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float e = __builtin_amdgcn_exp2f(fmaf(sacc[t][kb][i], c, -m_use));
          rs += e;
          pk[t][kb >> 1][(kb & 1) * 4 + i] = static_cast<__bf16>(e);
        }
      }
      l[t] = fmaf(l[t], alpha, rs);
      // the running max rarely moves after the first tiles: skip the rescale when no row
      // of this wave changed (wave-uniform branch)
      if (__any(alpha != 1.f)) {
#pragma unroll
        for (int db = 0; db < DB; ++db) o[t][db] *= alpha;
      }
    }

    // ---- O^T += V^T P^T ----
#pragma unroll
    for (int db = 0; db < DB; ++db) {
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const __bf16* base = &Vt[(db * 16 + lr) * VPAD + 32 * ks + 4 * lh];
        const uint2 lo = *reinterpret_cast<const uint2*>(base);
        const uint2 hi = *reinterpret_cast<const uint2*>(base + 16);
        const bf16x8 va = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
#pragma unroll
        for (int t = 0; t < TPW; ++t)
          if (tile_on[t])
            o[t][db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[t][ks], o[t][db], 0, 0, 0);
      }
    }
    __syncthreads();  // LDS tile consumed before the next one is staged
  }

  // ---- epilogue: normalise and store (final output, or split partials) ----
  const bool single = p.num_splits == 1;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    float lt = l[t];
    lt += __shfl_xor(lt, 16);
    lt += __shfl_xor(lt, 32);
    const int row = (qt0 + t) * 16 + lr;
    if (!tile_on[t] || row >= p.R) continue;
    const int node = row / p.g, head = hkv * p.g + row % p.g;
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse2 = lt > 0.f ? m[t] + log2f(lt) : -INFINITY;
    if (single) {
      uint16_t* out = static_cast<uint16_t*>(p.out) + (int64_t)b * p.o_sb +
                      (int64_t)node * p.o_sn + (int64_t)head * p.o_sh;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        bf16x4 v;
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = static_cast<__bf16>(o[t][db][i] * inv);
        *reinterpret_cast<bf16x4*>(out + db * 16 + 4 * lh) = v;
      }
      if (lh == 0 && p.lse) p.lse[((int64_t)b * p.N + node) * p.Hq + head] = lse2 * kLn2;
    } else {
      const int64_t prow = (((int64_t)b * p.Hkv + hkv) * p.num_splits + split) * p.R + row;
      float* dst = p.ws_o + prow * D;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(dst + db * 16 + 4 * lh) = o[t][db] * inv;
      if (lh == 0) p.ws_lse[prow] = lse2;
    }
  }
}

template <int D>
static hipError_t launch_d(const AttnParams& p, MfmaShape sh, hipStream_t s) {
  dim3 grid(p.num_splits, p.Hkv * p.row_chunks, p.B);
#define TV_CASE(TPW, NW)                                                             \
  if (sh.tpw == TPW && sh.nw == NW) {                                                \
    hipLaunchKernelGGL((tv_attn_mfma_kernel<D, TPW, NW>), grid, dim3(NW * 64), 0, s, p); \
    return hipGetLastError();                                                        \
  }
  TV_CASE(1, 1) TV_CASE(1, 2) TV_CASE(1, 3) TV_CASE(1, 4)
  TV_CASE(2, 3) TV_CASE(2, 4)
  TV_CASE(3, 3) TV_CASE(3, 4)
  TV_CASE(4, 3) TV_CASE(4, 4) TV_CASE(4, 8)
#undef TV_CASE
  return hipErrorInvalidConfiguration;
}

hipError_t launch_attn_mfma(const AttnParams& p, int D, MfmaShape shape, hipStream_t s) {
  return D == 64 ? launch_d<64>(p, shape, s) : launch_d<128>(p, shape, s);
}

}  // namespace tv
