// Causal prefill attention on CDNA4 matrix cores (gfx950) for the V2/V3 head
// shape: q [T, H, 192], k [Tk, H, 192] and v [Tk, H, 128] in bf16, o [T, H, 128], query row t
// at position q_off + t (Tk = q_off + T; q_off = 0 for a whole prefill, the cached prefix
// length for a chunk of a longer sequence):
//   o[t, h] = sum_{j <= q_off + t} softmax_j(scale * q[t,h] . k[j,h]) v[j,h]
// (NeMo "MLA" module: forward with a causal attention mask and softmax_scale).
//
// Flash-style: a workgroup owns 32*NW queries of one head and streams 64-key tiles
// of K and V through four LDS stages (direct global->LDS buffer copies, two tiles in
// flight, fence-free barriers).  Each wave
// keeps 32 queries: S^T = K Q^T with keys as the M dimension, so the softmax
// probabilities are already in the B-operand layout of O^T = V^T P^T; V^T is read
// with the transposing LDS read.  Online softmax in the log2 domain with a lazy
// rescale (the running max only moves when a tile exceeds it by 2^8).
// The kernel is persistent: one workgroup per CU walks a fixed list of (head, query
// tile) items.  Workgroup w runs on XCD w mod 8 (the dispatcher deals workgroups to the
// eight XCDs in turn), so heads h = x mod 8 are given to XCD x: its workgroups take that
// XCD's items head by head, query tiles heaviest first, dealt in serpentine order (round r
// takes items r*J .. r*J+J-1 of the XCD's list, reversed on odd rounds).  The workgroups'
// totals even out, and an XCD streams the K/V tiles of one or two heads at a time, which
// its L2 then serves to all of them.  Other grid or head counts use the same serpentine
// over the whole (query tile, head) list.
#include "mla_fast.h"

#include <algorithm>
#include <atomic>

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int DQK = 192, DV = 128;
constexpr int KC = DQK / 8, VC = DV / 8;   // 16-byte chunks per key / value row
constexpr int KT = 64;                     // keys per tile
constexpr int K_SLOTS = KT * KC, V_SLOTS = KT * VC;
constexpr float kRescaleThreshold = 8.0f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// K tile: key t, chunk c at slot KC*t + (c ^ k_swz(t)) (XOR inside aligned groups of 8).
// V tile: key t, chunk c at slot VC*t + (c ^ v_swz(t)).  Both keep the 16-lane passes of
// ds_read_b128 (score operand) and the 32-lane passes of ds_read_b64_tr_b16 (value
// operand) on distinct banks.
__device__ __forceinline__ int k_swz(int t) { return (t >> 1) & 7; }
__device__ __forceinline__ int v_swz(int t) { return 2 * (t & 7); }

struct PrefillArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  int T, H;
  int q_off, Tk;  // position of query row 0; keys (rows of k and v)
  float scale_log2;
  int n_qtiles;
};

// Copies of key tile kt: NW waves share K_SLOTS + V_SLOTS 16-byte slots, KI + VI per lane.
// Keys past Tk repeat the last key (their scores are masked).  Offsets are taken from the
// tile's first row of head h, so they stay far below 4 GB; a lane's offsets within a tile
// are the same for every tile but the last, so they are computed once (copy_offsets).
template <int NW>
struct CopyPlan {
  static constexpr int KI = K_SLOTS / 64 / NW, VI = V_SLOTS / 64 / NW;
  uint32_t off[KI + VI];
};

template <int NW>
__device__ __forceinline__ uint32_t copy_offset(const PrefillArgs& P, int i, int t_max, int w, int lane) {
  constexpr int KI = CopyPlan<NW>::KI, VI = CopyPlan<NW>::VI;
  if (i < KI) {
    const int p = 64 * (KI * w + i) + lane;
    const int t = p / KC, c = (p - t * KC) ^ k_swz(t);
    return (uint32_t)((min(t, t_max) * P.H * DQK + 8 * c) * 2);
  }
  const int p = 64 * (VI * w + (i - KI)) + lane;
  const int t = p / VC, c = (p - t * VC) ^ v_swz(t);
  return (uint32_t)((min(t, t_max) * P.H * DV + 8 * c) * 2);
}

template <int NW>
__device__ __forceinline__ CopyPlan<NW> copy_offsets(const PrefillArgs& P, int w, int lane) {
  CopyPlan<NW> cp;
#pragma unroll
  for (int i = 0; i < CopyPlan<NW>::KI + CopyPlan<NW>::VI; ++i) cp.off[i] = copy_offset<NW>(P, i, KT - 1, w, lane);
  return cp;
}

template <int NW>
__device__ __forceinline__ void issue_kv_copy(const PrefillArgs& P, int h, int kt, const CopyPlan<NW>& cp,
                                              uint4* __restrict__ kb, uint4* __restrict__ vb, int w, int lane) {
  constexpr int KI = CopyPlan<NW>::KI, VI = CopyPlan<NW>::VI;
  const int k0 = kt * KT, t_max = P.Tk - 1 - k0;
  const bf16_t* kbase = P.k + ((int64_t)k0 * P.H + h) * DQK;
  const bf16_t* vbase = P.v + ((int64_t)k0 * P.H + h) * DV;
  uint32_t off[KI + VI];
  if (t_max >= KT - 1) {
#pragma unroll
    for (int i = 0; i < KI + VI; ++i) off[i] = cp.off[i];
  } else {  // the tile runs past Tk
    int l = lane;
    asm volatile("" : "+v"(l));
#pragma unroll
    for (int i = 0; i < KI + VI; ++i) off[i] = copy_offset<NW>(P, i, t_max, w, l);
  }
#pragma unroll
  for (int i = 0; i < KI; ++i) dma16_buf(kbase, 0x7FFFFFF0u, off[i], kb + 64 * (KI * w + i));
#pragma unroll
  for (int i = 0; i < VI; ++i) dma16_buf(vbase, 0x7FFFFFF0u, off[KI + i], vb + 64 * (VI * w + i));
}

constexpr int kRing = 4;  // LDS operand reads in flight per wave in the matrix block

// Score operand i = 4*ks + mt (keys 16*mt .., dims 32*ks ..): slot KC*(16*mt + j) +
// ((4*ks + g) ^ k_swz(j)), the lane part in kbase[ks & 1].
__device__ __forceinline__ bf16x8 k_operand(const uint4* __restrict__ kb, const int (&kbase)[2], int i) {
  const int ks = i >> 2, mt = i & 3;
  return as_bf16x8(*(const uint4*)((const char*)kb + kbase[ks & 1] + (KC * 16 * mt + 8 * (ks >> 1)) * 16));
}

// Value operand i = 8*kk + mt (V^T rows 16*mt .., keys 32*kk ..): keys 32*kk + {0,16} + 4*g +
// j/4 (same swizzle), chunk 2*mt + half = (2*mt) ^ half, read with the transposing LDS read.
__device__ __forceinline__ bf16x8 v_operand(const uint4* __restrict__ vb, const int (&vbase)[4], int i) {
  const int kk = i >> 3, mt = i & 7;
  const char* pa = (const char*)vb + vbase[0] + (VC * 32 * kk) * 16 + ((2 * mt) ^ vbase[1]) * 16;
  const bf16x4 a0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)pa);
  const bf16x4 a1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(pa + VC * 16 * 16));
  return __builtin_shufflevector(a0, a1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Matrix block of one step for one wave: first this step's share of the K/V copies into the
// stage kn/vn, then (pv) O^T += V^T P^T for the previous tile from its probabilities pb, and
// (qk) S^T = K Q^T for the current tile.  Every LDS access of the step is issued here, through
// restrict pointers, so that the compiler's waits on the copies stay per access.
template <int NW>
__device__ __forceinline__ void mma_block(const PrefillArgs& P, int h, const CopyPlan<NW>& cp, bool copy, int kt_pf,
                                          bool qk, bool pv,
                                          const uint4* __restrict__ kb, const uint4* __restrict__ vb,
                                          uint4* __restrict__ kn, uint4* __restrict__ vn,
                                          const bf16x8 (&qf)[2][DQK / 32], f32x4 (&s)[4][2],
                                          const bf16x8 (&pb)[2][2], f32x4 (&o)[DV / 16][2], const int (&kbase)[2],
                                          const int (&vbase)[4], int w, int lane) {
  __builtin_amdgcn_s_setprio(1);  // this wave's matrix ops go first on the SIMD
  // the first score operands are read before the value product, which hides their latency
  // (unconditionally: a stage holds no tile the wave does not use yet, so such reads are
  // harmless and their results unused)
  bf16x8 kring[kRing];
#pragma unroll
  for (int i = 0; i < kRing; ++i) kring[i] = k_operand(kb, kbase, i);
  if (pv) {  // O^T[d][query] += V^T P^T; operand i = 8*kk + mt, kRing reads in flight
    bf16x8 ring[kRing];
#pragma unroll
    for (int i = 0; i < kRing; ++i) ring[i] = v_operand(vb, vbase, i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < 2 * DV / 16; ++i) {
      const int kk = i >> 3, mt = i & 7;
      const bf16x8 a = ring[i % kRing];
      if (i + kRing < 2 * DV / 16) ring[i % kRing] = v_operand(vb, vbase, i + kRing);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) o[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb[nt][kk], o[mt][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // S is written on every path (zeros for a tile the wave does not see), so the previous
  // tile's scores are dead during P V
  if (qk) {  // S^T[key][query]; operand i = 4*ks + mt, kRing reads in flight
    bf16x8 (&ring)[kRing] = kring;
#pragma unroll
    for (int i = 0; i < 4 * DQK / 32; ++i) {
      const int ks = i >> 2, mt = i & 3;
      const bf16x8 a = ring[i % kRing];
      if (i + kRing < 4 * DQK / 32) ring[i % kRing] = k_operand(kb, kbase, i + kRing);
#pragma unroll
      for (int nt = 0; nt < 2; ++nt)
        s[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[nt][ks], ks == 0 ? f32x4{0.f, 0.f, 0.f, 0.f} : s[mt][nt], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) s[mt][0] = s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // the copies go last, behind this step's LDS reads
  if (copy) issue_kv_copy<NW>(P, h, kt_pf, cp, kn, vn, w, lane);
  __builtin_amdgcn_s_setprio(0);
}

// Online softmax of one tile's scores (keys k0 .. k0+63) for the wave's 32 queries (lane's
// query at position qw0 + 16*nt + j): probabilities into pb (bf16, the B-operand layout of the value
// product), running max and sum updated, O rescaled when the max moves.  Every query sees
// key 0 in tile 0, so the running max is finite from the first tile on.  The max is taken
// over the raw scores and scaled afterwards (the scale is positive).
__device__ __forceinline__ void softmax_block(const PrefillArgs& P, int k0, int qw0, const f32x4 (&s)[4][2],
                                              bf16x8 (&pb)[2][2], f32x4 (&o)[DV / 16][2], float (&m_run)[2],
                                              float (&l_run)[2], int g, int j) {
  // both query groups side by side, with short dependency chains: one wave runs this alone on
  // its SIMD's vector ALU while the other wave's matrix ops run
  float x[2][4][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) x[nt][mt][i] = s[mt][nt][i];
  if (k0 + KT - 1 > qw0) {  // causal mask inside the diagonal tiles only
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = qw0 + 16 * nt + j;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (k0 + 16 * mt + 4 * g + i > qi) x[nt][mt][i] = -INFINITY;
    }
  }
  float m_new[2], corr[2];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    float mm[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) mm[mt] = fmaxf(fmaxf(x[nt][mt][0], x[nt][mt][1]), fmaxf(x[nt][mt][2], x[nt][mt][3]));
    const float mx = xmax16_32(fmaxf(fmaxf(mm[0], mm[1]), fmaxf(mm[2], mm[3]))) * P.scale_log2;
    m_new[nt] = (m_run[nt] == -INFINITY || mx > m_run[nt] + kRescaleThreshold) ? mx : m_run[nt];
    corr[nt] = m_run[nt] == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run[nt] - m_new[nt]);
  }
  float sum[2][4];
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      float p[8];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][2 * kk][i], P.scale_log2, -m_new[nt]));
        p[4 + i] = __builtin_amdgcn_exp2f(__builtin_fmaf(x[nt][2 * kk + 1][i], P.scale_log2, -m_new[nt]));
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[nt][i] = (kk == 0 ? 0.f : sum[nt][i]) + (p[i] + p[4 + i]);
      pb[nt][kk] = as_bf16x8(make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])));
    }
  }
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) {
    l_run[nt] = l_run[nt] * corr[nt] + xsum16_32((sum[nt][0] + sum[nt][1]) + (sum[nt][2] + sum[nt][3]));
    m_run[nt] = m_new[nt];
  }
  if (__any(corr[0] != 1.f || corr[1] != 1.f)) {
#pragma unroll
    for (int mt = 0; mt < DV / 16; ++mt) {
      o[mt][0] *= corr[0];
      o[mt][1] *= corr[1];
    }
  }
}

// Probabilities of a tile the wave does not see: written so that pb is dead between its use
// in the matrix block and the next softmax.
__device__ __forceinline__ void pb_clear(bf16x8 (&pb)[2][2]) {
#pragma unroll
  for (int nt = 0; nt < 2; ++nt) pb[nt][0] = pb[nt][1] = as_bf16x8(make_uint4(0u, 0u, 0u, 0u));
}

// K/V tiles in LDS: tile t in stage t mod 4.  Step t reads K of tile t and V of tile t-1 and
// copies tile t+2, into the stage of tile t-2, which step t-1 finished with.
constexpr int kStages = 4;

// Steps -2 .. n_kt of one item for a wave of group GRP (see prefill_attn_kernel); qw0 is the
// position of the wave's first query.
template <int NW, int GRP>
__device__ __forceinline__ void item_steps(const PrefillArgs& P, const CopyPlan<NW>& cp, int h, int n_kt, int qw0,
                                           uint4 (*kbuf)[K_SLOTS],
                                           uint4 (*vbuf)[V_SLOTS], const bf16x8 (&qf)[2][DQK / 32],
                                           f32x4 (&o)[DV / 16][2], float (&m_run)[2], float (&l_run)[2],
                                           const int (&kbase)[2], const int (&vbase)[4], int w, int lane) {
  const int g = lane >> 4, j = lane & 15;
  f32x4 s[4][2];
  bf16x8 pb[2][2];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) s[mt][0] = s[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  pb_clear(pb);
  constexpr int kCopies = (K_SLOTS + V_SLOTS) / 64 / NW;  // per wave per tile
  typedef __attribute__((address_space(3))) uint4 lds_uint4;
  // steps -2 and -1 only put tiles 0 and 1 in flight; step n_kt only adds P V of the last tile
  for (int kt = -2; kt <= n_kt; ++kt) {
    if (kt >= 0 && kt < n_kt) {
      // copies issued after tile kt's: those of tile kt+1, if any
      if (kt + 1 < n_kt) __builtin_amdgcn_s_waitcnt(0x0F70 | kCopies);
      else __builtin_amdgcn_s_waitcnt(0x0F70);
    }
    lds_barrier();
    const int kt_pf = kt + 2;
    const bool copy = kt_pf < n_kt;
    const bool qk = kt >= 0 && kt < n_kt && kt * KT <= qw0 + 31;    // this wave's queries see tile kt
    const bool pv = kt >= 1 && (kt - 1) * KT <= qw0 + 31;           // ... and tile kt-1
    // opaque copies of the stage pointers keep the restrict scopes of mma_block's parameters
    lds_uint4 *kc = (lds_uint4*)kbuf[kt & 3], *vp = (lds_uint4*)vbuf[(kt + 3) & 3];
    lds_uint4 *kn = (lds_uint4*)kbuf[kt_pf & 3], *vn = (lds_uint4*)vbuf[kt_pf & 3];
    asm volatile("" : "+s"(kc), "+s"(vp), "+s"(kn), "+s"(vn));
    if constexpr (GRP == 0) {
      mma_block<NW>(P, h, cp, copy, kt_pf, qk, pv, (const uint4*)kc, (const uint4*)vp, (uint4*)kn, (uint4*)vn, qf, s,
                    pb, o, kbase, vbase, w, lane);
      lds_barrier();
      if (qk) softmax_block(P, kt * KT, qw0, s, pb, o, m_run, l_run, g, j);
      else pb_clear(pb);
    } else {
      if (pv) softmax_block(P, (kt - 1) * KT, qw0, s, pb, o, m_run, l_run, g, j);
      else pb_clear(pb);
      lds_barrier();
      mma_block<NW>(P, h, cp, copy, kt_pf, qk, pv, (const uint4*)kc, (const uint4*)vp, (uint4*)kn, (uint4*)vn, qf, s,
                    pb, o, kbase, vbase, w, lane);
    }
  }
}

// Two waves share each SIMD.  Every step has two phases separated by a barrier: in the first,
// one wave of each pair (group 0) runs its matrix block while the other (group 1) runs its
// softmax; in the second they swap.  Group 0's step t: matrix block (S of tile t, O += P V of
// tile t-1), barrier, softmax of tile t.  Group 1's step t: softmax of tile t-1, barrier,
// matrix block (S of tile t, O += P V of tile t-1).  So the matrix cores and the vector ALUs
// of a SIMD work at the same time.
template <int NW>
__global__ __launch_bounds__(64 * NW, 1) void prefill_attn_kernel(PrefillArgs P) {
  __shared__ __attribute__((aligned(16))) uint4 kbuf[kStages][K_SLOTS];
  __shared__ __attribute__((aligned(16))) uint4 vbuf[kStages][V_SLOTS];
  constexpr int BQ = 32 * NW;
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  int grp;
  {  // group: the wave's rank, mod 2, among the waves of this workgroup on its SIMD (HW_ID bits 5:4)
    const int simd = (int)((__builtin_amdgcn_s_getreg(0x0904)) & 3);
    int* ids = (int*)&kbuf[0][0];
    if (lane == 0) ids[w] = simd;
    __syncthreads();
    int c = 0;
    for (int v = 0; v < w; ++v) c += ids[v] == simd;
    grp = __builtin_amdgcn_readfirstlane(c & 1);
    __syncthreads();
  }
  int kbase[2], vbase[4];
  {
    const int sj = k_swz(j);
#pragma unroll
    for (int e = 0; e < 2; ++e) kbase[e] = (KC * j + ((4 * e + g) ^ sj)) * 16;
    const int tA = 4 * g + (j >> 2), half = (j >> 1) & 1;
    vbase[0] = VC * tA * 16 + (j & 1) * 8;   // row part
    vbase[1] = half ^ v_swz(tA);            // chunk XOR
    vbase[2] = vbase[3] = 0;
  }
  const CopyPlan<NW> cp = copy_offsets<NW>(P, w, lane);
  const bool by_xcd = (gridDim.x & 7) == 0 && (P.H & 7) == 0;
  const int J = by_xcd ? (int)gridDim.x >> 3 : (int)gridDim.x;       // workgroups sharing one list
  const int slot = by_xcd ? (int)blockIdx.x >> 3 : (int)blockIdx.x;  // this workgroup's place in it
  const int n_list = by_xcd ? (P.H >> 3) * P.n_qtiles : P.H * P.n_qtiles;
  for (int r = 0; r * J < n_list; ++r) {
    const int m = r * J + ((r & 1) ? J - 1 - slot : slot);
    if (m >= n_list) continue;
    int h, qt;
    if (by_xcd) {  // XCD list: heads x, x + 8, ... one after another, query tiles heaviest first
      const int hi = m / P.n_qtiles;
      h = 8 * hi + ((int)blockIdx.x & 7);
      qt = P.n_qtiles - 1 - (m - hi * P.n_qtiles);
    } else {       // whole list: query tiles heaviest first, heads within
      h = m % P.H;
      qt = P.n_qtiles - 1 - m / P.H;
    }
    const int q0 = qt * BQ, qw0 = q0 + 32 * w;  // rows of q and o
    const int q_last = min(P.T, q0 + BQ) - 1;
    const int n_kt = (P.q_off + q_last) / KT + 1;
    bf16x8 qf[2][DQK / 32];
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = min(qw0 + 16 * nt + j, P.T - 1);
      const bf16_t* qrow = P.q + ((int64_t)qi * P.H + h) * DQK + 8 * g;
#pragma unroll
      for (int ks = 0; ks < DQK / 32; ++ks) qf[nt][ks] = as_bf16x8(*(const uint4*)(qrow + 32 * ks));
    }
    f32x4 o[DV / 16][2];
#pragma unroll
    for (int mt = 0; mt < DV / 16; ++mt) o[mt][0] = o[mt][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    float m_run[2] = {-INFINITY, -INFINITY}, l_run[2] = {0.f, 0.f};
    // the query fragments are complete before the loop, so no read in it waits for the copies
    __builtin_amdgcn_s_waitcnt(0);
    // one loop per group, so that each has its own register liveness
    const int qp0 = P.q_off + qw0;  // position of the wave's first query
    if (grp == 0) item_steps<NW, 0>(P, cp, h, n_kt, qp0, kbuf, vbuf, qf, o, m_run, l_run, kbase, vbase, w, lane);
    else item_steps<NW, 1>(P, cp, h, n_kt, qp0, kbuf, vbuf, qf, o, m_run, l_run, kbase, vbase, w, lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = qw0 + 16 * nt + j;
      if (qi >= P.T) continue;
      const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
      bf16_t* dst = P.o + ((int64_t)qi * P.H + h) * DV + 4 * g;
#pragma unroll
      for (int mt = 0; mt < DV / 16; ++mt) {
        const f32x4 v = o[mt][nt] * inv;
        *(uint2*)(dst + 16 * mt) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
    // every wave is done with the last tiles' stages before the next item's copies refill them
    lds_barrier();
  }
}

}  // namespace

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cached[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
    cached[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

bool fast_prefill_attn_supported(const Dims& d) {
  return d.act == 1 && d.dn + d.dr == DQK && d.dv == DV && d.scale > 0.f;
}

size_t fast_prefill_attn_ws_bytes(const Dims&, int) { return 0; }

hipError_t fast_prefill_attn(const Dims& d, const void* q, const void* k, const void* v, int T, void* o, void* ws,
                             hipStream_t s) {
  return fast_prefill_attn_offset(d, q, k, v, T, 0, o, ws, s);
}

hipError_t fast_prefill_attn_offset(const Dims& d, const void* q, const void* k, const void* v, int T, int q_off,
                                    void* o, void*, hipStream_t s) {
  PrefillArgs P;
  P.q = (const bf16_t*)q;
  P.k = (const bf16_t*)k;
  P.v = (const bf16_t*)v;
  P.o = (bf16_t*)o;
  P.T = T;
  P.H = d.H;
  P.q_off = q_off;
  P.Tk = q_off + T;
  P.scale_log2 = d.scale * 1.4426950408889634f;
  // one workgroup per CU (the four K/V stages take all 160 KB of a CU's LDS).  256 queries per
  // workgroup (8 waves, two per SIMD playing ping-pong) unless the items are then too few and
  // uneven to share out: the larger of the heaviest item and the mean load per workgroup must
  // stay within 1.25x the mean; else 128 queries (4 waves)
  const int cus = device_cu_count();
  const int nq8 = (T + 255) / 256;
  int64_t sum8 = 0;
  for (int i = 0; i < nq8; ++i) sum8 += (q_off + std::min(T, 256 * (i + 1)) - 1) / KT + 1;
  const int64_t max8 = (q_off + T - 1) / KT + 1;
  const int64_t items8 = (int64_t)d.H * nq8;
  const double mean8 = (double)sum8 * d.H / (double)std::min<int64_t>(items8, cus);
  const bool big = (double)std::max<int64_t>(max8, 1) <= 1.25 * mean8;
  const int BQ = big ? 256 : 128;
  P.n_qtiles = (T + BQ - 1) / BQ;
  const int total = d.H * P.n_qtiles;
  const int grid = std::min(total, cus);
  if (big) prefill_attn_kernel<8><<<grid, 512, 0, s>>>(P);
  else prefill_attn_kernel<4><<<grid, 256, 0, s>>>(P);
  return hipGetLastError();
}

}  // namespace mla
