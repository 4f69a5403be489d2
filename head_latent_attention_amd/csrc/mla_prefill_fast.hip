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
#include <vector>

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

// Work items of one head, heaviest first: a query tile, or one part of its key tiles when a
// query tile alone would leave the workgroups uneven (the parts write partial results that
// prefill_merge_kernel combines).  Entry: query tile (bits 0-9), part (10-12), parts (13-15),
// partial-result slot within the head (16-31).
constexpr int kMaxItemsPerHead = 256;

struct PrefillArgs {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;
  bf16_t* o;
  int T, H;
  int q_off, Tk;  // position of query row 0; keys (rows of k and v)
  float scale_log2;
  int n_qtiles;
  int n_items;               // entries of items per head; 0: whole query tiles, heaviest first
  int cost_major;            // XCD lists ordered by item cost across the XCD's heads (few rounds)
  int slots_per_head;        // partial-result slots per head
  float* part_o;             // [H][slots_per_head][BQ][DV] fp32, normalised by its own sum
  float* part_ml;            // [H][slots_per_head][BQ][2]  (running max, log2 units; sum)
  uint32_t items[kMaxItemsPerHead];
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
    // no scores: the registers are only redefined (no instructions), so that the previous
    // tile's scores are dead here; the softmax does not read them on this path
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      asm volatile("" : "=v"(s[mt][0]));
      asm volatile("" : "=v"(s[mt][1]));
    }
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
    // two chains of three-input maxima over the lane's 16 scores (8 instructions)
    float ma = fmaxf(fmaxf(x[nt][0][0], x[nt][0][1]), x[nt][0][2]);
    float mb = fmaxf(fmaxf(x[nt][2][0], x[nt][2][1]), x[nt][2][2]);
    ma = fmaxf(fmaxf(ma, x[nt][0][3]), x[nt][1][0]);
    mb = fmaxf(fmaxf(mb, x[nt][2][3]), x[nt][3][0]);
    ma = fmaxf(fmaxf(ma, x[nt][1][1]), x[nt][1][2]);
    mb = fmaxf(fmaxf(mb, x[nt][3][1]), x[nt][3][2]);
    const float mx = xmax16_32(fmaxf(fmaxf(ma, x[nt][1][3]), fmaxf(mb, x[nt][3][3]))) * P.scale_log2;
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

// Steps -2 .. n_kt of one item (key tiles kt0 .. kt0 + n_kt - 1) for a wave of group GRP (see
// prefill_attn_kernel); qw0 is the position of the wave's first query.
template <int NW, int GRP>
__device__ __forceinline__ void item_steps(const PrefillArgs& P, const CopyPlan<NW>& cp, int h, int kt0, int n_kt,
                                           int qw0,
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
    const bool qk = kt >= 0 && kt < n_kt && (kt0 + kt) * KT <= qw0 + 31;  // this wave's queries see tile kt
    const bool pv = kt >= 1 && (kt0 + kt - 1) * KT <= qw0 + 31;         // ... and tile kt-1
    // opaque copies of the stage pointers keep the restrict scopes of mma_block's parameters
    lds_uint4 *kc = (lds_uint4*)kbuf[kt & 3], *vp = (lds_uint4*)vbuf[(kt + 3) & 3];
    lds_uint4 *kn = (lds_uint4*)kbuf[kt_pf & 3], *vn = (lds_uint4*)vbuf[kt_pf & 3];
    asm volatile("" : "+s"(kc), "+s"(vp), "+s"(kn), "+s"(vn));
    if constexpr (GRP == 0) {
      mma_block<NW>(P, h, cp, copy, kt0 + kt_pf, qk, pv, (const uint4*)kc, (const uint4*)vp, (uint4*)kn, (uint4*)vn,
                    qf, s, pb, o, kbase, vbase, w, lane);
      lds_barrier();
      if (qk) softmax_block(P, (kt0 + kt) * KT, qw0, s, pb, o, m_run, l_run, g, j);
      else pb_clear(pb);
    } else {
      if (pv) softmax_block(P, (kt0 + kt - 1) * KT, qw0, s, pb, o, m_run, l_run, g, j);
      else pb_clear(pb);
      lds_barrier();
      mma_block<NW>(P, h, cp, copy, kt0 + kt_pf, qk, pv, (const uint4*)kc, (const uint4*)vp, (uint4*)kn, (uint4*)vn,
                    qf, s, pb, o, kbase, vbase, w, lane);
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
  const int per_head = P.n_items > 0 ? P.n_items : P.n_qtiles;
  const int n_list = by_xcd ? (P.H >> 3) * per_head : P.H * per_head;
  for (int r = 0; r * J < n_list; ++r) {
    const int m = r * J + ((r & 1) ? J - 1 - slot : slot);
    if (m >= n_list) continue;
    int h, e;
    if (by_xcd) {  // XCD list: heads x, x + 8, ... one after another, items heaviest first
      // (with few rounds, heaviest first across those heads instead)
      const int hx = P.H >> 3;
      const int hi = P.cost_major ? m % hx : m / per_head;
      h = 8 * hi + ((int)blockIdx.x & 7);
      e = P.cost_major ? m / hx : m - hi * per_head;
    } else {       // whole list: items heaviest first, heads within
      h = m % P.H;
      e = m / P.H;
    }
    int qt = P.n_qtiles - 1 - e, part = 0, parts = 1, pslot = 0;
    if (P.n_items > 0) {
      const uint32_t ent = P.items[e];
      qt = (int)(ent & 0x3FF);
      part = (int)((ent >> 10) & 7);
      parts = (int)((ent >> 13) & 7);
      pslot = (int)(ent >> 16);
    }
    const int q0 = qt * BQ, qw0 = q0 + 32 * w;  // rows of q and o
    const int q_last = min(P.T, q0 + BQ) - 1;
    const int n_all = (P.q_off + q_last) / KT + 1;
    // part p of `parts` covers key tiles [b_p, b_(p+1)): every boundary lies below the tiles the
    // query tile's first row cannot see whole, so each part's first tile is visible to all rows
    const int n_full = (P.q_off + q0) / KT;
    auto bound = [&](int p) { return p == 0 ? 0 : (p >= parts ? n_all : min(p * n_all / parts, n_full - 1)); };
    const int kt0 = bound(part), n_kt = bound(part + 1) - kt0;
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
    if (grp == 0) item_steps<NW, 0>(P, cp, h, kt0, n_kt, qp0, kbuf, vbuf, qf, o, m_run, l_run, kbase, vbase, w, lane);
    else item_steps<NW, 1>(P, cp, h, kt0, n_kt, qp0, kbuf, vbuf, qf, o, m_run, l_run, kbase, vbase, w, lane);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) {
      const int qi = qw0 + 16 * nt + j;
      if (qi >= P.T) continue;
      const float inv = l_run[nt] > 0.f ? 1.f / l_run[nt] : 0.f;
      if (parts > 1) {  // a part: fp32 output normalised by its own sum, running max and sum
        const int64_t row = ((int64_t)h * P.slots_per_head + pslot) * BQ + (qi - q0);
        float* dst = P.part_o + row * DV + 4 * g;
#pragma unroll
        for (int mt = 0; mt < DV / 16; ++mt) *(f32x4*)(dst + 16 * mt) = o[mt][nt] * inv;
        if (g == 0) *(float2*)(P.part_ml + row * 2) = make_float2(m_run[nt], l_run[nt]);
        continue;
      }
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

// Query tiles whose key tiles were split into parts: entry = query tile (bits 0-9), parts
// (10-12), first partial-result slot within the head (16-31).
struct MergeArgs {
  const float* part_o;
  const float* part_ml;
  bf16_t* o;
  int T, H, BQ, slots_per_head;
  uint32_t tiles[kMaxItemsPerHead];
};

// o[q, h] of a split query tile from its parts: each part's output (normalised by its own sum
// l_p, running max m_p in log2 units) weighted by 2^(m_p - M) * l_p, M the largest m_p, in part
// order.  One thread per (row, four value columns); grid (split tiles x heads, BQ * DV / 4 / 256).
__global__ __launch_bounds__(256) void prefill_merge_kernel(MergeArgs M) {
  const int th = blockIdx.x, tile = th / M.H, h = th - tile * M.H;
  const uint32_t ent = M.tiles[tile];
  const int qt = (int)(ent & 0x3FF), parts = (int)((ent >> 10) & 7), slot0 = (int)(ent >> 16);
  const int e = blockIdx.y * 256 + threadIdx.x, r = e / (DV / 4), c = e - r * (DV / 4);
  const int qi = qt * M.BQ + r;
  if (r >= M.BQ || qi >= M.T) return;
  const int64_t row0 = ((int64_t)h * M.slots_per_head + slot0) * M.BQ + r;
  float mx = -INFINITY;
  for (int p = 0; p < parts; ++p) mx = fmaxf(mx, M.part_ml[(row0 + (int64_t)p * M.BQ) * 2]);
  f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
  float wsum = 0.f;
  for (int p = 0; p < parts; ++p) {
    const int64_t row = row0 + (int64_t)p * M.BQ;
    const float2 ml = *(const float2*)(M.part_ml + row * 2);
    const float wgt = __builtin_amdgcn_exp2f(ml.x - mx) * ml.y;
    acc += *(const f32x4*)(M.part_o + row * DV + 4 * c) * wgt;
    wsum += wgt;
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  acc *= inv;
  *(uint2*)(M.o + ((int64_t)qi * M.H + h) * DV + 4 * c) = make_uint2(pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]));
}

// Launch plan of the prefill attention: 256 queries per workgroup (8 waves) unless the work
// items are then too uneven; on the 8-wave path with no query offset, query tiles whose key
// tiles exceed the mean load per workgroup are split into up to four parts of whole key tiles
// (partials merged afterwards), so that few heads or short sequences still fill every CU.
struct PrefillPlan {
  bool big = true, cost_major = false;
  int BQ = 256, n_qtiles = 0;
  std::vector<uint32_t> items;  // empty: whole query tiles, heaviest first
  std::vector<uint32_t> split_tiles;
  int slots_per_head = 0;
  size_t ws_bytes = 0;
};

PrefillPlan prefill_plan(const Dims& d, int T, int q_off, bool allow_split, int cus) {
  PrefillPlan pl;
  const int nq = (T + 255) / 256;
  auto tiles_of = [&](int i) { return (q_off + std::min(T, 256 * (i + 1)) - 1) / KT + 1; };
  int64_t total = 0;
  for (int i = 0; i < nq; ++i) total += tiles_of(i);
  total *= d.H;
  std::vector<int> parts(nq, 1);
  if (allow_split) {
    // parts of at most 3/4 of the mean load per workgroup (a finer cut evens out the last round)
    const int64_t target = std::max<int64_t>(3 * ((total + cus - 1) / cus) / 4, 16);
    for (int i = 0; i < nq; ++i) {
      const int n_full = (q_off + 256 * i) / KT, c = tiles_of(i);
      if (c > target && n_full >= 2) parts[i] = (int)std::min<int64_t>({4, (c + target - 1) / target, n_full});
    }
  }
  // entries (cost, query tile, part), with the kernel's part boundaries
  struct Ent { int cost, qt, part, parts; };
  std::vector<Ent> ents;
  bool any_split = false;
  for (int i = 0; i < nq; ++i) {
    const int n_all = tiles_of(i), n_full = (q_off + 256 * i) / KT, np = parts[i];
    auto bound = [&](int p) { return p == 0 ? 0 : (p >= np ? n_all : std::min(p * n_all / np, n_full - 1)); };
    for (int p = 0; p < np; ++p) ents.push_back({bound(p + 1) - bound(p), i, p, np});
    any_split |= np > 1;
  }
  std::stable_sort(ents.begin(), ents.end(), [](const Ent& a, const Ent& b) {
    return a.cost != b.cost ? a.cost > b.cost : a.qt > b.qt;
  });
  int max_item = 0;
  for (const Ent& e : ents) max_item = std::max(max_item, e.cost);
  const int64_t n_items = (int64_t)d.H * (int64_t)ents.size();
  const double mean = (double)total / (double)std::min<int64_t>(n_items, cus);
  pl.big = (double)std::max(max_item, 1) <= 1.25 * mean;
  if (!pl.big) {  // 128 queries per workgroup, whole query tiles
    pl.BQ = 128;
    pl.n_qtiles = (T + 127) / 128;
    return pl;
  }
  pl.n_qtiles = nq;
  if (!any_split || ents.size() > (size_t)kMaxItemsPerHead) return pl;
  {  // rounds of an XCD's list: with few, order it by cost rather than head by head
    const int grid = (int)std::min<int64_t>(n_items, cus);
    if (grid % 8 == 0 && d.H % 8 == 0) {
      const int64_t J = grid / 8, list = (int64_t)(d.H / 8) * (int64_t)ents.size();
      pl.cost_major = (list + J - 1) / J <= 4;
    }
  }
  // partial-result slots: the parts of each split query tile, consecutive
  std::vector<int> slot0(nq, -1);
  for (int i = 0; i < nq; ++i)
    if (parts[i] > 1) {
      slot0[i] = pl.slots_per_head;
      pl.split_tiles.push_back((uint32_t)i | ((uint32_t)parts[i] << 10) | ((uint32_t)pl.slots_per_head << 16));
      pl.slots_per_head += parts[i];
    }
  for (const Ent& e : ents) {
    const int sl = e.parts > 1 ? slot0[e.qt] + e.part : 0;
    pl.items.push_back((uint32_t)e.qt | ((uint32_t)e.part << 10) | ((uint32_t)e.parts << 13) | ((uint32_t)sl << 16));
  }
  pl.ws_bytes = (size_t)d.H * pl.slots_per_head * pl.BQ * (DV * 4 + 8);
  return pl;
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

size_t fast_prefill_attn_ws_bytes(const Dims& d, int T) {
  if (!fast_prefill_attn_supported(d) || T <= 0) return 0;
  return prefill_plan(d, T, 0, true, device_cu_count()).ws_bytes;
}

hipError_t fast_prefill_attn(const Dims& d, const void* q, const void* k, const void* v, int T, void* o, void* ws,
                             hipStream_t s) {
  return fast_prefill_attn_offset(d, q, k, v, T, 0, o, ws, s);
}

hipError_t fast_prefill_attn_offset(const Dims& d, const void* q, const void* k, const void* v, int T, int q_off,
                                    void* o, void* ws, hipStream_t s) {
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
  // one workgroup per CU (the four K/V stages take all 160 KB of a CU's LDS)
  const int cus = device_cu_count();
  const PrefillPlan pl = prefill_plan(d, T, q_off, q_off == 0 && ws != nullptr, cus);
  P.n_qtiles = pl.n_qtiles;
  P.n_items = (int)pl.items.size();
  P.cost_major = pl.cost_major ? 1 : 0;
  P.slots_per_head = pl.slots_per_head;
  P.part_o = (float*)ws;
  P.part_ml = ws ? (float*)((char*)ws + (size_t)d.H * pl.slots_per_head * pl.BQ * DV * 4) : nullptr;
  for (size_t i = 0; i < pl.items.size(); ++i) P.items[i] = pl.items[i];
  const int per_head = P.n_items > 0 ? P.n_items : P.n_qtiles;
  const int grid = std::min(d.H * per_head, cus);
  if (pl.big) prefill_attn_kernel<8><<<grid, 512, 0, s>>>(P);
  else prefill_attn_kernel<4><<<grid, 256, 0, s>>>(P);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || pl.split_tiles.empty()) return e;
  MergeArgs M;
  M.part_o = P.part_o;
  M.part_ml = P.part_ml;
  M.o = P.o;
  M.T = T;
  M.H = d.H;
  M.BQ = pl.BQ;
  M.slots_per_head = pl.slots_per_head;
  for (size_t i = 0; i < pl.split_tiles.size(); ++i) M.tiles[i] = pl.split_tiles[i];
  prefill_merge_kernel<<<dim3((unsigned)pl.split_tiles.size() * d.H, pl.BQ * (DV / 4) / 256), 256, 0, s>>>(M);
  return hipGetLastError();
}

}  // namespace mla
