// Tree-verify attention, VALU path: fp32 inputs, or bf16 when the packed rows of one
// (request, kv head) -- N nodes x (Hq/Hkv) query heads -- do not fill a 16-row matrix tile.
//
// Semantics ("Tree attention mask for draft-tree verification", "A strong answer";
// "Tree Verification", "Tree Attention"): packed row r = node * g + j (g = Hq/Hkv) is query
// head hkv*g + j of tree node r / g.  It attends every prefix key t < L and tree key
// L + i exactly when bit i of the node's ancestor bitmask is set.  The bitmask is built in
// LDS from the parent array, never read as a dense mask.
//
// One workgroup = (key split, kv head x row chunk, request); 4 waves, 4 packed rows each.
// Keys stream through LDS in 64-key tiles converted to fp32 (16-byte loads, all of a tile's
// issued before any is stored); lane = key for the scores, lane = feature for P.V; online
// softmax in the exp2 domain with wave reductions.
#include "kernels_common.h"

namespace tv {

template <typename T>
__device__ inline float load_elem(const T* p);
template <>
__device__ inline float load_elem<float>(const float* p) { return *p; }
template <>
__device__ inline float load_elem<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// The 16-byte chunk `c` (four fp32 or eight bf16 values) unpacked to fp32.
template <typename T>
__device__ inline void unpack16(const uint4& c, float* out);
template <>
__device__ inline void unpack16<float>(const uint4& c, float* out) {
  out[0] = __uint_as_float(c.x);
  out[1] = __uint_as_float(c.y);
  out[2] = __uint_as_float(c.z);
  out[3] = __uint_as_float(c.w);
}
template <>
__device__ inline void unpack16<uint16_t>(const uint4& c, float* out) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

template <typename T>
__device__ inline void store_elem(T* p, float v);
template <>
__device__ inline void store_elem<float>(float* p, float v) { *p = v; }
template <>
__device__ inline void store_elem<uint16_t>(uint16_t* p, float v) { *p = f32_to_bf16(v); }

template <typename T, int D>
__global__ void __launch_bounds__(256) tv_attn_valu_kernel(AttnParams p) {
  constexpr int KT = kKeysPerTile;
  constexpr int ROWS = kValuRowsPerWg;
  constexpr int RPW = ROWS / 4;  // rows per wave
  constexpr int E = D / 64;      // features per lane
  __shared__ float Ks[KT][D + 1];
  __shared__ float Vs[KT][D];
  __shared__ float Qs[ROWS][D];
  __shared__ float Ps[4][KT];
  __shared__ double inv_s[D / 2];  // rotary pair frequencies, formed once per workgroup
  __shared__ uint64_t mask_s[TV_MAX_NODES];
  __shared__ int32_t par_s[TV_MAX_NODES];

  const int split = blockIdx.x;
  const int hkv = blockIdx.y % p.Hkv;
  const int rc = blockIdx.y / p.Hkv;
  const int b = blockIdx.z;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int L = clamped_prefix(p, b);
  const int Ttot = L + p.N;
  const int kbeg = split * p.chunk;
  if (kbeg >= Ttot) return;  // this request has fewer splits
  const int kend = min(kbeg + p.chunk, Ttot);

  const T* __restrict__ q = static_cast<const T*>(p.q);
  const T* __restrict__ kp = static_cast<const T*>(p.k);
  const T* __restrict__ vp = static_cast<const T*>(p.v);

  // parent links staged in LDS: the walks below then take no global round trip per level
  if (tid < p.N) par_s[tid] = p.parent[(int64_t)b * p.parent_sb + tid];
  __syncthreads();
  if (tid < p.N) {
    bool ok;
    int dd;
    const uint64_t m = ancestor_bits(par_s, tid, p.N, ok, dd);
    mask_s[tid] = m;
    // one workgroup per request (split 0, first row chunk of kv head 0) exports the tree
    if (blockIdx.x == 0 && blockIdx.y == 0) export_node_meta(p, b, tid, m, ok, dd);
  }
  for (int idx = tid; idx < ROWS * D; idx += 256) {
    const int r = idx / D, d = idx - (idx / D) * D;
    const int row = rc * ROWS + r;
    float val = 0.f;
    if (row < p.R) {
      const int node = row / p.g, head = hkv * p.g + row % p.g;
      val = load_elem<T>(q + (int64_t)b * p.q_sb + (int64_t)node * p.q_sn +
                         (int64_t)head * p.q_sh + d);
    }
    Qs[r][d] = val;
  }
  if (p.rope)
    for (int i = tid; i < D / 2; i += 256) inv_s[i] = rope_inv_freq(i, D, p.rope_log2_theta);
  __syncthreads();
  if (p.rope) {  // fused rotary embedding of the queries at L + depth (uniform branch)
    for (int idx = tid; idx < ROWS * (D / 2); idx += 256) {
      const int r = idx / (D / 2), mm = idx - (idx / (D / 2)) * (D / 2);
      const int row = rc * ROWS + r;
      if (row >= p.R) continue;
      float cs, sn;
      rope_cos_sin_inv(L + depth_of(mask_s[row / p.g]), inv_s[mm], cs, sn);
      rope_pair(Qs[r][mm], Qs[r][mm + D / 2], cs, sn);
    }
    __syncthreads();
  }

  float m[RPW], l[RPW], o[RPW][E];
  uint64_t rmask[RPW];
  bool rvalid[RPW];
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const int row = rc * ROWS + w * RPW + j;
    rvalid[j] = row < p.R;
    rmask[j] = rvalid[j] ? mask_s[row / p.g] : 0ull;
    m[j] = -INFINITY;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[j][e] = 0.f;
  }

  // a tile's K and V as 16-byte chunks (strides and bases are 16-byte multiples), every
  // load of the tile issued before any of them is stored to LDS
  constexpr int VE = 16 / sizeof(T);            // elements per chunk
  constexpr int CPR = D / VE;                   // chunks per row
  constexpr int PER = KT * CPR / 256;           // chunks per thread, K and V each
  static_assert(KT * CPR % 256 == 0, "tile chunks split evenly over the workgroup");
  for (int kt0 = kbeg; kt0 < kend; kt0 += KT) {
    uint4 kc[PER], vc[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i;
      const int t = kt0 + c / CPR;
      kc[i] = vc[i] = make_uint4(0, 0, 0, 0);
      if (t < kend) {
        const int64_t off = kv_offset(p, b, t, hkv) + (c % CPR) * VE;
        kc[i] = *reinterpret_cast<const uint4*>(kp + off);
        vc[i] = *reinterpret_cast<const uint4*>(vp + off);
      }
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int c = tid + 256 * i;
      const int key = c / CPR, d0 = (c % CPR) * VE;
      float kf[VE], vf[VE];
      unpack16<T>(kc[i], kf);
      unpack16<T>(vc[i], vf);
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        Ks[key][d0 + e] = kf[e];
        Vs[key][d0 + e] = vf[e];
      }
    }
    __syncthreads();
    if (p.rope && kt0 + KT > L) {  // tile holds tree keys: rotate them at L + depth
      for (int idx = tid; idx < KT * (D / 2); idx += 256) {
        const int key = idx / (D / 2), mm = idx - (idx / (D / 2)) * (D / 2);
        const int t = kt0 + key;
        if (t < L || t >= kend) continue;
        float cs, sn;
        rope_cos_sin_inv(L + depth_of(mask_s[t - L]), inv_s[mm], cs, sn);
        rope_pair(Ks[key][mm], Ks[key][mm + D / 2], cs, sn);
      }
      __syncthreads();
    }
    const int t = kt0 + lane;
    const bool in_range = t < kend;
#pragma unroll
    for (int j = 0; j < RPW; ++j) {
      if (!rvalid[j]) continue;  // wave-uniform
      const float* qr = Qs[w * RPW + j];
      float s = 0.f;
#pragma unroll 8
      for (int d = 0; d < D; ++d) s = fmaf(qr[d], Ks[lane][d], s);
      const int off = t - L;
      const bool allowed =
          in_range && (t < L || ((rmask[j] >> (off & 63)) & 1ull));
      s = allowed ? s * p.scale_log2 : -INFINITY;
      const float mx = wave_max(s);
      const float m_new = fmaxf(m[j], mx);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2f(m[j] - m_use);
      const float pj = exp2f(s - m_use);
      l[j] = l[j] * alpha + pj;
      Ps[w][lane] = pj;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int d = lane + 64 * e;
        float acc = 0.f;
#pragma unroll 8
        for (int key = 0; key < KT; ++key) acc = fmaf(Ps[w][key], Vs[key][d], acc);
        o[j][e] = fmaf(o[j][e], alpha, acc);
      }
      __builtin_amdgcn_wave_barrier();
      m[j] = m_new;
    }
    __syncthreads();
  }

  const bool single = single_split(p, Ttot);
#pragma unroll
  for (int j = 0; j < RPW; ++j) {
    const float lsum = wave_sum(l[j]);
    if (!rvalid[j]) continue;
    const int row = rc * ROWS + w * RPW + j;
    const int node = row / p.g, head = hkv * p.g + row % p.g;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    const float lse2 = lsum > 0.f ? m[j] + log2f(lsum) : -INFINITY;
    if (single) {
      T* out = static_cast<T*>(p.out) + (int64_t)b * p.o_sb + (int64_t)node * p.o_sn +
               (int64_t)head * p.o_sh;
#pragma unroll
      for (int e = 0; e < E; ++e) store_elem<T>(out + lane + 64 * e, o[j][e] * inv);
      if (lane == 0 && p.lse)
        p.lse[((int64_t)b * p.N + node) * p.Hq + head] = lse2 * kLn2;
    } else {
      const int64_t prow =
          (((int64_t)b * p.Hkv + hkv) * p.num_splits + split) * p.R + row;
#pragma unroll
      for (int e = 0; e < E; ++e) p.ws_o[prow * D + lane + 64 * e] = o[j][e] * inv;
      if (lane == 0) p.ws_lse[prow] = lse2;
    }
  }
}

hipError_t launch_attn_valu(const AttnParams& p, int D, bool bf16, hipStream_t s) {
  dim3 grid(p.num_splits, p.Hkv * p.row_chunks, p.B);
  dim3 block(256);
  if (bf16) {
    if (D == 64)
      hipLaunchKernelGGL((tv_attn_valu_kernel<uint16_t, 64>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((tv_attn_valu_kernel<uint16_t, 128>), grid, block, 0, s, p);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((tv_attn_valu_kernel<float, 64>), grid, block, 0, s, p);
    else
      hipLaunchKernelGGL((tv_attn_valu_kernel<float, 128>), grid, block, 0, s, p);
  }
  return hipGetLastError();
}

}  // namespace tv
