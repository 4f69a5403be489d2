// Absorbed MLA decode attention on CDNA4 matrix cores (gfx950), for the
// DeepSeek-V2/V3 head geometry: 128 heads, kv_lora 512, qk_rope 64, qk_nope 128,
// v_dim 128, bf16 activations and cache, bf16 or block-scaled E4M3FN weights.
//
// Three kernels; the first also plans:
//   plan     prefix sums of 64-token tiles over the batch (the work list), by one extra
//            workgroup of the fold launch.
//   fold     q_lat[b,h] = q_nope[b,h] @ W_UK[h], W_UK read straight out of wkv_b
//            (AWS NKI "MLA Decode QKV Kernel API Reference": the query is absorbed
//            into the cache's latent space; atlas "Struct MlaWeights": w_uk_t).
//   attn     split-context attention: the concatenated tile list is cut into 256
//            equal shares, one workgroup each.  A workgroup streams its rows of
//            [c_kv | k_pe] (576 bf16) into LDS once (direct global->LDS copies, three
//            sub-tiles ahead in four rotating buffers) for all 128 heads and keeps an
//            unnormalised latent output, running max and sum per head.
//   combine  log-sum-exp merge of the shares of each sequence, then the value
//            extraction o = o_lat @ W_UV[h] (atlas "Struct MlaWeights": w_uv).
//
// Matrix-core layout of the attention (8 waves, 16 heads each):
//   S^T = K Q^T with tokens as the M dimension (A operand read from LDS with
//   ds_read_b128) and heads as N (Q^T held in registers for the whole segment).
//   The S^T accumulator already has the lane layout of the B operand of
//   O^T = V^T P^T, so probabilities go from the softmax straight into the PV
//   matrix op; V^T comes from the same row-major LDS tile with the gfx950
//   transposing read ds_read_b64_tr_b16.  Rows are XOR-swizzled in 16-byte
//   chunks so both read patterns are bank-conflict free.
#include "mla_fast.h"

#include <type_traits>

namespace mla {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr int kH = 128, kLkv = 512, kDr = 64, kR = 576, kDn = 128, kDv = 128;
constexpr int kChunks = kR / 8;   // 16-byte chunks per cache row
constexpr int kTile = 64;         // tokens per work-list tile
constexpr int kSub = 32;          // tokens per LDS buffer of the attention kernel
constexpr int kAttnWGs = 256;     // workgroups of the attention kernel (one per CU on MI355X)
constexpr int kXcds = 8;          // MI355X: accelerator dies, each with its own L2

// Share of the work list taken by attention workgroup wg.  Workgroups are dealt to the
// dies round-robin (wg % 8), so die x gets shares [32x, 32x + 32): workgroups that split
// a sequence mostly sit on one die and fetch its query through the same L2.
__device__ __forceinline__ int wg_share(int wg) {
  return (wg % kXcds) * (kAttnWGs / kXcds) + wg / kXcds;
}
constexpr float kRescaleThreshold = 8.0f;  // log2 units: p = 2^(s - m) <= 256 between rescales


__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }

// Eight consecutive weight elements (k fixed, n..n+7) as bf16; fp8 codes are
// converted exactly (E4M3FN value times a power-of-two block scale).
template <int WK>
__device__ __forceinline__ uint4 load_w8(const WeightView& W, int64_t k, int64_t n) {
  if constexpr (WK == W_BF16) {
    return *(const uint4*)((const bf16_t*)W.w + k * W.ld + n);
  } else {
    const uint2 raw = *(const uint2*)((const uint8_t*)W.w + k * W.ld + n);
    const float s = W.scale[(k >> 7) * W.scale_ld + (n >> 7)];
    uint32_t out[4];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint32_t word = h ? raw.y : raw.x;
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)word, true);
      out[2 * h] = pack_bf16x2(lo[0] * s, lo[1] * s);
      out[2 * h + 1] = pack_bf16x2(hi[0] * s, hi[1] * s);
    }
    return make_uint4(out[0], out[1], out[2], out[3]);
  }
}

// ------------------------------------------------------------------------------ plan
// P[b] = number of 64-token tiles of sequences 0..b-1; P[B] = total.  Then, for each share r
// of the attention work list (tiles [r*N/G, (r+1)*N/G)), info[2r] = its first sequence with
// tokens in the share (B when empty) and info[2r+1] = its number of 32-token sub-tiles, so
// that no attention workgroup walks P with chains of dependent scalar loads.
__device__ __forceinline__ int share_tokens(const int32_t* P, const int32_t* ctx, int b,
                                            int t_lo, int t_hi, int* lo, int* hi) {
  const int p0 = P[b], p1 = P[b + 1];
  const int a = max(t_lo, p0), e = min(t_hi, p1);
  if (a >= e) return 0;
  *lo = (a - p0) * kTile;
  *hi = min(ctx[b], (e - p0) * kTile);
  return 1;
}

constexpr int kPlanLds = 2048;  // batches up to this size are planned out of LDS

constexpr int kPlanThreads = 256;
static_assert(kAttnWGs == kPlanThreads, "one planning thread per attention share");

// Run by one 256-thread workgroup (the last workgroup of the fold launch).
__device__ void plan_block(const int32_t* __restrict__ ctx, int B, int32_t* __restrict__ P, int32_t* __restrict__ info,
                           bf16_t* __restrict__ zero_row, int32_t* scan, int32_t* Ps, int32_t* Cs) {
  const int tid = threadIdx.x;
  const bool in_lds = B <= kPlanLds;
  for (int i = tid; i < kR; i += kPlanThreads) zero_row[i] = 0;
  if (tid == 0) {
    P[0] = 0;
    Ps[0] = 0;
  }
  // P[b + 1] = P[b] + tiles of sequence b, 256 sequences per round (inclusive scan in LDS)
  int carry = 0;
  for (int c0 = 0; c0 < B; c0 += kPlanThreads) {
    const int b = c0 + tid;
    const int c = b < B ? ctx[b] : 0;
    scan[tid] = c > 0 ? (c + kTile - 1) / kTile : 0;
    __syncthreads();
    for (int off = 1; off < kPlanThreads; off <<= 1) {
      const int v = tid >= off ? scan[tid - off] : 0;
      __syncthreads();
      scan[tid] += v;
      __syncthreads();
    }
    if (b < B) {
      P[b + 1] = carry + scan[tid];
      if (in_lds) {
        Ps[b + 1] = carry + scan[tid];
        Cs[b] = c;
      }
    }
    carry += scan[kPlanThreads - 1];
    __syncthreads();
  }
  __syncthreads();  // P (global) and Ps are read by other threads of this workgroup below
  const int32_t* PP = in_lds ? Ps : P;
  const int32_t* CC = in_lds ? Cs : ctx;
  const int N = carry;
  const int t_lo = (int)((int64_t)tid * N / kAttnWGs), t_hi = (int)((int64_t)(tid + 1) * N / kAttnWGs);
  int first = B, total = 0;
  if (t_lo < t_hi) {
    // the largest b with P[b] <= t_lo
    int l = 0, h = B;
    while (l < h) {
      const int mid = (l + h + 1) >> 1;
      if (PP[mid] <= t_lo) l = mid;
      else h = mid - 1;
    }
    for (int b = l; b < B && PP[b] < t_hi; ++b) {
      int a, e;
      if (!share_tokens(PP, CC, b, t_lo, t_hi, &a, &e)) continue;
      if (first == B) first = b;
      total += (e - a + kSub - 1) / kSub;
    }
  }
  info[2 * tid] = first;
  info[2 * tid + 1] = total;
}

// ------------------------------------------------------------------------------ fold
// Qabs[b][h] = [q_nope[b][h] @ W_UK[h] | q_pe[b][h]] in bf16, W_UK[h][p][c] = wkv_b[c][h*256 + p].
// Grid (H + 1, 4, ceil(B / 256)): workgroup (h, cg, z) covers latent columns [128cg, 128cg + 128)
// of rows [256z, 256z + 256), wave w the 32 columns [128cg + 32w, 128cg + 32w + 32); its W_UK
// operands are loaded once and kept in registers while it walks its rows in groups of 64 (so
// W_UK is read once per 256 rows).  Every operand load of a group is issued before its first
// matrix op.
template <int WK>
__global__ __launch_bounds__(256) void fold_kernel(const bf16_t* __restrict__ q, int B, WeightView W,
                                                   bf16_t* __restrict__ Qabs, const int32_t* __restrict__ ctx,
                                                   int32_t* __restrict__ P, int32_t* __restrict__ info,
                                                   bf16_t* __restrict__ zero_row) {
  if (blockIdx.x == kH) {  // one extra workgroup plans the attention's work list
    __shared__ int32_t scan[kPlanThreads];
    __shared__ int32_t Ps[kPlanLds + 1];
    __shared__ int32_t Cs[kPlanLds];
    if (blockIdx.y == 0 && blockIdx.z == 0) plan_block(ctx, B, P, info, zero_row, scan, Ps, Cs);
    return;
  }
  __shared__ __attribute__((aligned(16))) uint4 tile[64 * 16];  // 64 rows x 128 columns, bf16
  const int h = blockIdx.x, cg = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
  constexpr int qs = kH * (kDn + kDr);
  const int c0 = 128 * cg + 32 * w;
  uint4 bw[kDn / 32][2];
#pragma unroll
  for (int ks = 0; ks < kDn / 32; ++ks)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      bw[ks][nt] = load_w8<WK>(W, c0 + 16 * nt + j, (int64_t)h * (kDn + kDv) + 32 * ks + 8 * g);
  bf16_t* tb = (bf16_t*)tile;
  const int b_end = min(B, 256 * (int)blockIdx.z + 256);
  for (int b0 = 256 * (int)blockIdx.z; b0 < b_end; b0 += 64) {
    uint4 a[kDn / 32][4];
    // every load is issued unconditionally (rows past B repeat row B - 1 and are never stored),
    // so all of them are in flight together
#pragma unroll
    for (int ks = 0; ks < kDn / 32; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int b = min(b0 + 16 * mt + j, B - 1);
        a[ks][mt] = *(const uint4*)(q + (size_t)b * qs + h * (kDn + kDr) + 32 * ks + 8 * g);
      }
    __builtin_amdgcn_sched_barrier(0);  // keep every load above the first matrix op
    f32x4 acc[4][2];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) acc[mt][nt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < kDn / 32; ++ks)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 2; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a[ks][mt]), as_bf16x8(bw[ks][nt]),
                                                                acc[mt][nt], 0, 0, 0);
    if (b0 > 256 * (int)blockIdx.z) __syncthreads();  // the previous group's stores have read the tile
    // the 64 x 128 result through LDS (16-byte chunks, chunk c of row r at slot 16r + (c ^ (r & 15)))
    // so that each row goes out as 16-byte stores
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * mt + 4 * g + i;
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const int c = 32 * w + 16 * nt + j;
          tb[(16 * r + ((c >> 3) ^ (r & 15))) * 8 + (c & 7)] = f32_to_bf16(acc[mt][nt][i]);
        }
      }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + tid, r = e >> 4, ch = e & 15, b = b0 + r;
      if (b < B) *(uint4*)(Qabs + ((size_t)b * kH + h) * kR + 128 * cg + 8 * ch) = tile[16 * r + (ch ^ (r & 15))];
    }
    // rope part of the query is carried over unchanged
    if (cg == 0) {
      for (int e = tid; e < 64 * kDr / 8; e += 256) {
        const int r = e / (kDr / 8), c = e - r * (kDr / 8), b = b0 + r;
        if (b < B)
          *(uint4*)(Qabs + ((size_t)b * kH + h) * kR + kLkv + 8 * c) =
              *(const uint4*)(q + (size_t)b * qs + h * (kDn + kDr) + kDn + 8 * c);
      }
    }
  }
}

// ------------------------------------------------------------------------------ attention
// LDS tile of 32 tokens: region C holds the 512 latent values of each token as
// 64 chunks of 16 bytes (token t, chunk c at slot 64*t + (c ^ swz_c(t))), region
// PE the 64 rope values as 8 chunks (slot 8*t + (c ^ swz_pe(t))).  gfx950 serves a
// 64-lane ds_read_b128 in four passes of 16 lanes, the lanes of a pass being the
// lane quads of equal bit parity within each half wave, and a ds_read_b64_tr_b16
// in two passes of 32 lanes; a pass is conflict-free when its lanes hit distinct
// 4-byte banks.  swz_c (linear in the token's low 4 bits) satisfies both the
// 16-token score reads and the 4-token transposing value reads; swz_pe the score
// reads of the rope chunks.  Four such buffers rotate: three tiles of
// copies are in flight while the fourth is being consumed.
constexpr int kCSlots = kSub * 64, kPeSlots = kSub * 8, kBufSlots = kCSlots + kPeSlots;
constexpr int kNBuf = 4;
constexpr int kAttnWaves = 8;
static_assert(kTile % kSub == 0, "work-list tiles are whole LDS buffers");

__device__ __forceinline__ int swz_c(int t) { return ((t & 7) << 1) ^ (((t >> 3) & 1) * 9); }
__device__ __forceinline__ int swz_pe(int t) { return (t >> 1) & 7; }

struct AttnArgs {
  const bf16_t* Qabs;
  const bf16_t* cache;
  const bf16_t* zero_row;  // kR zeros: source of rows past the context or with an invalid block id
  int64_t n_blocks;
  int bs;
  const int32_t* bt;
  int max_blocks;
  int64_t bt_stride;  // elements between the table rows of consecutive sequences (0: one shared row)
  const int32_t* ctx;
  const int32_t* P;
  const int32_t* info;  // per share: first sequence, number of sub-tiles
  int B;
  float scale_log2;
  bf16_t* part_o;  // [(G + B)][H/16][Lkv/64][16][64]  latent output of a share, normalised by its own sum
  float* part_ml;  // [(G + B)][H][2]    (running max in log2 units, sum)
};

// Wave-uniform load through the scalar cache (the value is read-only for the kernel's lifetime).
template <typename T>
__device__ __forceinline__ T sload(const T* p) {
  return *(const __attribute__((address_space(4))) T*)p;
}

// Block id of the (block-size aligned) 32-token sub-tile starting at token tok0, or -1.
__device__ __forceinline__ int sub_tile_block(const AttnArgs& A, int b, int tok0, int tok_hi) {
  if (tok0 >= tok_hi) return -1;
  const int lb = tok0 / A.bs;
  return lb < A.max_blocks ? sload(A.bt + (size_t)b * A.bt_stride + lb) : -1;
}

// Direct global->LDS copies of one 32-token sub-tile of block `blk`.  The block size is a
// multiple of 32, so the sub-tile's rows are 32 consecutive rows of one cache block.  Wave
// w copies the latent parts of tokens [4w, 4w + 4) (one 64-lane copy each); waves 0..3
// also copy the rope parts of tokens [8w, 8w + 8) (8 lanes per token).  Latent parts of
// rows past the context, and all of an invalid block, come from the zero row: the value
// product multiplies them by a zero probability, which must not meet a NaN.
__device__ __forceinline__ void issue_tile_copy(const AttnArgs& A, int blk, int tok0, int tok_hi,
                                                uint4* __restrict__ buf, int w, int lane) {
  const bool blk_ok = blk >= 0 && blk < A.n_blocks;
  const bf16_t* base = A.cache + ((int64_t)blk * A.bs + (tok0 % A.bs)) * kR;
  int l = lane;
  asm volatile("" : "+v"(l));
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = 4 * w + i;
    const bf16_t* row = (blk_ok && tok0 + t < tok_hi) ? base + t * kR : A.zero_row;  // wave-uniform
    dma16_buf(row, kR * 2, 16 * (l ^ swz_c(t)), buf + 64 * t);
  }
  if (w < 4) {
    // rope parts of tokens [8w, 8w + 8), 8 lanes each.  Rows past the context but inside the
    // block are copied as they are: only the scores read them, and those are masked.
    const int t0 = 8 * w, t = t0 + (l >> 3);
    const bf16_t* slab = blk_ok ? base + t0 * kR : A.zero_row;  // wave-uniform
    const uint32_t row = blk_ok ? (uint32_t)(l >> 3) : 0u;
    dma16_buf(slab, blk_ok ? 8 * kR * 2 : kR * 2, row * kR * 2 + kLkv * 2 + 16 * ((l & 7) ^ swz_pe(t)),
              buf + kCSlots + 64 * w);
  }
}

// Waits until this wave's copies of the oldest in-flight sub-tile have landed, given
// that `later` further sub-tiles' copies were issued after it.
__device__ __forceinline__ void wait_copies(int w, int later) {
  // copies per sub-tile per wave: 5 for waves 0..3, 4 for waves 4..7
  if (w < 4) {
    if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 10);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 5);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  } else {
    if (later >= 2) __builtin_amdgcn_s_waitcnt(0x0F70 | 8);
    else if (later == 1) __builtin_amdgcn_s_waitcnt(0x0F70 | 4);
    else __builtin_amdgcn_s_waitcnt(0x0F70);
  }
}

// Byte offsets, within an LDS buffer, of this lane's operand chunks.  (4*ks + g) ^ swz_c(j) equals
// 16*(ks >> 2) + ((4*(ks & 3) + g) ^ swz_c(j)) as swz_c < 16, so four lane offsets plus immediates
// cover the 16 latent k-steps of the score reads (two more the rope k-steps); likewise
// (2*mt) ^ vU = 16*(mt >> 3) + ((2*(mt & 7)) ^ vU) leaves eight offsets for the value reads.
struct LaneOffsets {
  int s[4], pe[2], v[8];
};

__device__ __forceinline__ LaneOffsets lane_offsets(int lane) {
  const int g = lane >> 4, j = lane & 15;
  LaneOffsets L;
  const int sj = swz_c(j), pj = swz_pe(j);
#pragma unroll
  for (int q = 0; q < 4; ++q) L.s[q] = (64 * j + ((4 * q + g) ^ sj)) * 16;
#pragma unroll
  for (int q = 0; q < 2; ++q) L.pe[q] = (kCSlots + 8 * j + ((4 * q + g) ^ pj)) * 16;
  // value reads: tokens {0,16} + 4*g + j/4 share the swizzle of 4*g + j/4; chunk 2*mt + half
  const int tA = 4 * g + (j >> 2);
  const int vU = ((j >> 1) & 1) ^ swz_c(tA);
#pragma unroll
  for (int q = 0; q < 8; ++q) L.v[q] = 64 * tA * 16 + (j & 1) * 8 + ((2 * q) ^ vU) * 16;
  return L;
}

constexpr int kSPre = 4;  // score operand reads in flight per wave
constexpr int kVPre = 4;  // value operand reads in flight per wave

// V^T operand of latent tile mt (16 latent rows x 32 tokens) by two transposing reads.
__device__ __forceinline__ bf16x8 v_read(const char* bbase, const LaneOffsets& LO, int mt) {
  const char* q = bbase + LO.v[mt & 7] + 256 * (mt >> 3);
  const bf16x4 b0 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)q);
  const bf16x4 b1 = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)(q + 16 * 64 * 16));
  return __builtin_shufflevector(b0, b1, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Scores of one sub-tile for this wave's 16 heads, then the online softmax (log2 domain,
// lazy rescale of the running output).  Returns P^T as the B operand of the value product.
// The first two value operand reads are issued before the softmax, which reads no LDS, so
// that their latency is hidden behind it (more would not fit in the registers).
__device__ __forceinline__ bf16x8 scores_softmax(const AttnArgs& A, int tok0, int tok_hi, const char* bbase,
                                                 const LaneOffsets& LO, const bf16x8 (&qf)[kR / 32],
                                                 f32x4 (&o)[kLkv / 16], float& m_run, float& l_run,
                                                 bf16x8 (&vring)[kVPre], int lane) {
  const int g = lane >> 4;
  // ---- S^T[token][head]: 2 token tiles of 16; k-steps 0..15 latent, 16..17 rope
  auto s_read = [&](int it) -> bf16x8 {
    const int ks = it >> 1, mt = it & 1;
    if (ks < 16) return as_bf16x8(*(const uint4*)(bbase + LO.s[ks & 3] + 256 * (ks >> 2) + 16 * 64 * 16 * mt));
    return as_bf16x8(*(const uint4*)(bbase + LO.pe[ks - 16] + 16 * 8 * 16 * mt));
  };
  constexpr int kSIt = 2 * (kR / 32);
  f32x4 s[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
  bf16x8 ring[kSPre];
#pragma unroll
  for (int it = 0; it < kSPre; ++it) ring[it] = s_read(it);
  // the program order below is the schedule: kSPre reads stay in flight ahead of the matrix ops
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int it = 0; it < kSIt; ++it) {
    s[it & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ring[it % kSPre], qf[it >> 1], s[it & 1], 0, 0, 0);
    if (it + kSPre < kSIt) ring[it % kSPre] = s_read(it + kSPre);
    __builtin_amdgcn_sched_barrier(0);
  }
#pragma unroll
  for (int mt = 0; mt < 2; ++mt) vring[mt] = v_read(bbase, LO, mt);
  __builtin_amdgcn_sched_barrier(0);
  // ---- online softmax; the lane's head is 16*w + j, its tokens 16*mt + 4*g + i
  float x[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[i] = s[0][i] * A.scale_log2;
    x[4 + i] = s[1][i] * A.scale_log2;
  }
  if (tok0 + kSub > tok_hi) {  // only the last sub-tile of a segment has tokens past the end
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (tok0 + 4 * g + i >= tok_hi) x[i] = -INFINITY;
      if (tok0 + 16 + 4 * g + i >= tok_hi) x[4 + i] = -INFINITY;
    }
  }
  float mx = x[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) mx = fmaxf(mx, x[i]);
  mx = xmax16_32(mx);
  const float m_new = (m_run == -INFINITY || mx > m_run + kRescaleThreshold) ? mx : m_run;
  const float corr = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
  float p[8];
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    p[i] = __builtin_amdgcn_exp2f(x[i] - m_new);
    sum += p[i];
  }
  const bf16x8 pb = as_bf16x8(make_uint4(pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                                         pack_bf16x2(p[6], p[7])));
  sum = xsum16_32(sum);
  l_run = l_run * corr + sum;
  m_run = m_new;
  if (__any(corr != 1.f)) {
#pragma unroll
    for (int mt = 0; mt < kLkv / 16; ++mt) o[mt] *= corr;
  }
  return pb;
}

// O^T[latent][head] += V^T P^T over one sub-tile's 32 tokens (one k-step per latent tile).
// vring holds the operands of latent tiles 0 and 1 on entry.
__device__ __forceinline__ void value_product(const char* bbase, const LaneOffsets& LO, const bf16x8& pb,
                                              f32x4 (&o)[kLkv / 16], bf16x8 (&vring)[kVPre]) {
#pragma unroll
  for (int mt = 2; mt < kVPre; ++mt) vring[mt] = v_read(bbase, LO, mt);
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < kLkv / 16; ++mt) {
    o[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vring[mt % kVPre], pb, o[mt], 0, 0, 0);
    if (mt + kVPre < kLkv / 16) vring[mt % kVPre] = v_read(bbase, LO, mt + kVPre);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Writes this wave's partial result (16 heads x 512 latents, normalised by l_run) as rows of
// 64 latents, the wave's 16 heads contiguous per quarter (part_o layout [pair][head group]
// [quarter][16][64]): lane (g, j) holds latents 16mt + 4g .. + 3 of head j; each quarter
// (tiles 4q .. 4q + 3) goes through the wave's LDS stage (row = head, 128 bytes; the 16-byte
// chunk c of row r at slot 8r + (c ^ (r & 7))) and out as two 1 KB stores of eight whole rows.
__device__ __forceinline__ void store_partial(bf16_t* part_o, size_t ps, int w, int lane, float l_run,
                                              const f32x4 (&o)[kLkv / 16], uint4* __restrict__ st) {
  int l = lane;
  asm volatile("" : "+v"(l));  // keeps the address arithmetic here, out of the main loop
  const int g = l >> 4, j = l & 15, hh = l >> 3, k = l & 7;
  const float inv_l = 1.f / l_run;
  char* stb = (char*)st;
#pragma unroll
  for (int q = 0; q < kLkv / 64; ++q) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int mt = 4 * q + t, c = 2 * t + (g >> 1);
      *(uint2*)(stb + (8 * j + (c ^ (j & 7))) * 16 + 8 * (g & 1)) =
          make_uint2(pack_bf16x2(o[mt][0] * inv_l, o[mt][1] * inv_l), pack_bf16x2(o[mt][2] * inv_l, o[mt][3] * inv_l));
    }
    const uint4 v0 = st[8 * hh + (k ^ (hh & 7))];
    const uint4 v1 = st[8 * (8 + hh) + (k ^ (hh & 7))];
    bf16_t* dq = part_o + ((ps * (kH / 16) + w) * (kLkv / 64) + q) * 16 * 64 + 8 * k;
    *(uint4*)(dq + 64 * hh) = v0;
    *(uint4*)(dq + 64 * (8 + hh)) = v1;
  }
}

// One step: the copies of a later sub-tile go into `nxt`; then, when `compute` is set, this
// wave takes sub-tile `cur` (tokens from tok0): scores, softmax and value product, and when
// `last` is set it writes the partial result of the sequence (pair slot ps) through `st`.  The
// buffers are restrict-qualified so that, once inlined, the copies into `nxt` carry alias
// scopes disjoint from the reads of `cur` and the accesses of `st`; every copy is issued by
// this one inlined call site, so the compiler never makes those LDS accesses wait for copies
// in flight.
__device__ __forceinline__ void attn_step(const AttnArgs& A, int tok0, int tok_hi, bool copy, int blk_pf, int tok_pf,
                                          int tok_hi_pf, bool compute, const uint4* __restrict__ cur,
                                          uint4* __restrict__ nxt, const LaneOffsets& LO, const bf16x8 (&qf)[kR / 32],
                                          f32x4 (&o)[kLkv / 16], float& m_run, float& l_run, int w, int lane,
                                          bool last, size_t ps, uint4* __restrict__ st) {
  if (copy) issue_tile_copy(A, blk_pf, tok_pf, tok_hi_pf, nxt, w, lane);
  if (!compute) return;
  bf16x8 vring[kVPre];
  const bf16x8 pb = scores_softmax(A, tok0, tok_hi, (const char*)cur, LO, qf, o, m_run, l_run, vring, lane);
  value_product((const char*)cur, LO, pb, o, vring);
  if (last) store_partial(A.part_o, ps, w, lane, l_run, o, st);
}

constexpr int kPf = 3;  // sub-tiles whose copies are issued ahead of the one being computed
static_assert(kNBuf >= kPf + 1, "buffers: the current one and the ones in flight");

// A position in a workgroup's share of the work list: sequence b, sub-tile starting at
// token tok, the share's part of sequence b ending at token tok_hi.
struct Cursor {
  int b, tok, tok_hi;
};

// Part of sequence b inside tiles [t_lo, t_hi): tokens [*lo, *hi); false when empty.
__device__ __forceinline__ bool share_of(const AttnArgs& A, int b, int t_lo, int t_hi, int* lo, int* hi) {
  const int p0 = sload(A.P + b), p1 = sload(A.P + b + 1);
  const int a = max(t_lo, p0), e = min(t_hi, p1);
  if (a >= e) return false;
  *lo = (a - p0) * kTile;
  *hi = min(sload(A.ctx + b), (e - p0) * kTile);
  return true;
}

// Moves c to the first sub-tile of the next non-empty sequence of the share (b = B when none).
// The walk stops at the first sequence that starts at or past the share's end, so that the
// end of a share costs one probe rather than a walk over the rest of the batch.
__device__ __forceinline__ void next_segment(const AttnArgs& A, int t_lo, int t_hi, Cursor& c) {
  for (++c.b; c.b < A.B; ++c.b) {
    if (sload(A.P + c.b) >= t_hi) break;
    if (share_of(A, c.b, t_lo, t_hi, &c.tok, &c.tok_hi)) return;
  }
  c.b = A.B;
}

__device__ __forceinline__ void advance(const AttnArgs& A, int t_lo, int t_hi, Cursor& c) {
  c.tok += kSub;
  if (c.tok >= c.tok_hi) next_segment(A, t_lo, t_hi, c);
}

// 512 threads = 8 waves; wave w owns heads [16w, 16w + 16).  The workgroup's share of the
// work list is one stream of 32-token sub-tiles across sequence boundaries: the copies run
// kPf sub-tiles ahead of the computation, also into the next sequence; at a boundary the
// finished sequence's partial result is written and the next sequence's query loaded (a
// wait that also covers the copies in flight).
__global__ __launch_bounds__(64 * kAttnWaves, 1) void decode_attn_kernel(AttnArgs A) {
  __shared__ __attribute__((aligned(16))) uint4 kv[kNBuf][kBufSlots];
  // per wave: 16 heads x 64 latents of a partial result on its way out (the rest of the LDS)
  __shared__ __attribute__((aligned(16))) uint4 stage[kAttnWaves][16 * 8];
  const int tid = threadIdx.x, lane = tid & 63, g = lane >> 4, j = lane & 15;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int N = sload(A.P + A.B);
  const int wg = wg_share(blockIdx.x);
  const int t_lo = (int)((int64_t)wg * N / kAttnWGs), t_hi = (int)((int64_t)(wg + 1) * N / kAttnWGs);
  const int total = sload(A.info + 2 * wg + 1);
  if (total == 0) return;
  Cursor cc{sload(A.info + 2 * wg), 0, 0};
  share_of(A, cc.b, t_lo, t_hi, &cc.tok, &cc.tok_hi);
  Cursor pc = cc;
  const int head = 16 * w + j;
  const LaneOffsets LO = lane_offsets(lane);
  // The loads complete before the function returns (an explicit wait for every memory
  // operation of the wave), so the compiler sees the fragments ready on every later step and
  // never waits for the copies in flight before a score product.
  auto load_q = [&](int b, bf16x8 (&qf)[kR / 32]) {
    const bf16_t* qrow = A.Qabs + ((size_t)b * kH + head) * kR + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kR / 32; ++ks) qf[ks] = as_bf16x8(*(const uint4*)(qrow + 32 * ks));
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
  };
  // Q^T fragments of this wave's 16 heads (B operand of S^T = K Q^T)
  bf16x8 qf[kR / 32];
  load_q(cc.b, qf);
  f32x4 o[kLkv / 16];
#pragma unroll
  for (int mt = 0; mt < kLkv / 16; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  // steps s < 0 only put the first kPf sub-tiles in flight
  for (int s = -kPf; s < total; ++s) {
    const bool copy = s + kPf < total;
    const int blk_pf = copy ? sub_tile_block(A, pc.b, pc.tok, pc.tok_hi) : -1;  // scalar load, overlaps the barrier
    if (s >= 0) {
      // copies issued after sub-tile s's: those of the next min(kPf - 1, ...) sub-tiles.  Other
      // memory operations issued in between (partial results, query loads) only make this
      // wait longer, never shorter.
      wait_copies(w, min(total - 1 - s, kPf - 1));
      lds_barrier();
    }
    const bool last = s >= 0 && cc.tok + kSub >= cc.tok_hi;  // last sub-tile of sequence cc.b
    attn_step(A, cc.tok, cc.tok_hi, copy, blk_pf, pc.tok, pc.tok_hi, s >= 0, kv[s < 0 ? 0 : s % kNBuf],
              kv[(s + kPf + kNBuf) % kNBuf], LO, qf, o, m_run, l_run, w, lane, last, (size_t)wg + cc.b, stage[w]);
    if (copy) advance(A, t_lo, t_hi, pc);
    if (s < 0) continue;
    if (cc.tok + kSub < cc.tok_hi) {
      cc.tok += kSub;
      continue;
    }
    // ---- last sub-tile of sequence cc.b: its partial result went out in the step; the
    // running max and sum follow
    const size_t ps = (size_t)wg + cc.b;
    if (g == 0) *(float2*)(A.part_ml + (ps * kH + head) * 2) = make_float2(m_run, l_run);
    next_segment(A, t_lo, t_hi, cc);
    if (cc.b >= A.B) break;
    load_q(cc.b, qf);
#pragma unroll
    for (int mt = 0; mt < kLkv / 16; ++mt) o[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run = -INFINITY;
    l_run = 0.f;
  }
}

// Work-list share of attention workgroup w: tiles [w*N/G, (w+1)*N/G).
__device__ __forceinline__ bool wg_nonempty(int w, int N) {
  return (int64_t)w * N / kAttnWGs < (int64_t)(w + 1) * N / kAttnWGs;
}

// ------------------------------------------------------------------------------ combine + W_UV
// Grid (H, ceil(B/16)).  Merges the partials of 16 sequences for one head, then
// o[b][h] = o_lat[b][h] @ W_UV[h] on the matrix cores (W_UV[h][c][j] = wkv_b[c][h*256 + 128 + j]).
// A share's weight in the merge is 2^(m - M) * l (its normalised output times its own sum),
// accumulated online (running max M) in share order.  All of W_UV[h] is loaded into registers
// before the merge, so that its latency overlaps the merge's loads.
template <int WK, int SG>
__global__ __launch_bounds__(256) void combine_kernel(const bf16_t* __restrict__ part_o,
                                                      const float* __restrict__ part_ml, const int32_t* __restrict__ P,
                                                      int B, WeightView W, bf16_t* __restrict__ out) {
  // merged latent rows As [16 SG][512] and one 64-row chunk of W_UV[h] Ws [64][128], bf16, both
  // unpadded with 16-byte chunks XOR-swizzled by row (As: chunk c of row r at 64r + (c ^ (r & 15));
  // Ws: chunk c of row r at 16r + (c ^ ws_swz(r))), so that four groups of 16 sequences take
  // 80 KB and two workgroups fit on a CU
  __shared__ __attribute__((aligned(16))) uint4 As[16 * SG * (kLkv / 8)];
  __shared__ __attribute__((aligned(16))) uint4 Ws[64 * (kDv / 8)];
  const int h = blockIdx.x, b0 = blockIdx.y * 16 * SG;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, g = lane >> 4, j = lane & 15;
  const int N = P[B];
  const int64_t col0 = (int64_t)h * (kDn + kDv) + kDn;
  // the rows of a 32-lane transposing read (8 rows: 4 consecutive, twice, 8 apart) get distinct
  // even keys, so each row's 32 bytes land on their own banks
  auto ws_swz = [](int r) { return 2 * ((r & 3) + 4 * ((r >> 3) & 1)); };
  // W_UV[h] in eight chunks of 64 rows, two in registers at a time: the first two load ahead of
  // the merge, each later one once the chunk two before it is in LDS; every chunk serves all SG
  // groups of 16 sequences
  constexpr int AH = 2, kWc = kLkv / 64;
  uint4 wr[AH][4];
  auto load_chunk = [&](int cc) {
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + tid, r = e >> 4, ch = e & 15;
      wr[cc % AH][it] = load_w8<WK>(W, 64 * cc + r, col0 + 8 * ch);
    }
  };
#pragma unroll
  for (int cc = 0; cc < AH; ++cc) load_chunk(cc);
  __builtin_amdgcn_sched_barrier(0);  // the weight loads stay ahead of the merge
  // ---- merge: the 16 lanes of quarter g of wave w handle local row 4w + g of each group, each
  // lane 32 latent columns, so the four rows of a wave run their shares side by side (four
  // shares per round)
  for (int sg = 0; sg < SG; ++sg) {
    const int lb = 16 * sg + 4 * w + g, b = b0 + lb;
    float acc[32];
#pragma unroll
    for (int e = 0; e < 32; ++e) acc[e] = 0.f;
    int wf = 0, wl = -1;
    if (b < B) {
      const int p0 = P[b], p1 = P[b + 1];
      if (p1 > p0) {
        wf = (int)(((int64_t)(p0 + 1) * kAttnWGs - 1) / N);
        wl = (int)(((int64_t)p1 * kAttnWGs - 1) / N);
      }
    }
    float M = -INFINITY, L = 0.f;
    for (int wq0 = wf; wq0 <= wl; wq0 += 4) {
      float2 ml[4];
      uint4 v[4][4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int wq = wq0 + u;
        ok[u] = wq <= wl && wg_nonempty(wq, N);
        const size_t pp = (size_t)(ok[u] ? wq : wf) + b;
        const size_t ps = pp * kH + h;
        // latents 32j .. 32j + 31 of head h: half (j & 1) of its row in quarter j / 2
        const size_t pq = (((pp * (kH / 16) + (h >> 4)) * (kLkv / 64) + (j >> 1)) * 16 + (h & 15)) * 64 + 32 * (j & 1);
        ml[u] = *(const float2*)(part_ml + ps * 2);
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) v[u][q4] = *(const uint4*)(part_o + pq + 8 * q4);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (!ok[u]) continue;  // an empty share's slot was never written
        const float Mn = fmaxf(M, ml[u].x);
        const float sa = M == -INFINITY ? 0.f : exp2f(M - Mn);
        const float f = exp2f(ml[u].x - Mn) * ml[u].y;
        L = L * sa + f;
        M = Mn;
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const uint32_t wds[4] = {v[u][q4].x, v[u][q4].y, v[u][q4].z, v[u][q4].w};
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            acc[8 * q4 + 2 * e] = acc[8 * q4 + 2 * e] * sa + f * __uint_as_float(wds[e] << 16);
            acc[8 * q4 + 2 * e + 1] = acc[8 * q4 + 2 * e + 1] * sa + f * __uint_as_float(wds[e] & 0xFFFF0000u);
          }
        }
      }
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4)
      As[lb * (kLkv / 8) + ((4 * j + q4) ^ (lb & 15))] =
          make_uint4(pack_bf16x2(acc[8 * q4] * inv, acc[8 * q4 + 1] * inv),
                     pack_bf16x2(acc[8 * q4 + 2] * inv, acc[8 * q4 + 3] * inv),
                     pack_bf16x2(acc[8 * q4 + 4] * inv, acc[8 * q4 + 5] * inv),
                     pack_bf16x2(acc[8 * q4 + 6] * inv, acc[8 * q4 + 7] * inv));
  }
  // ---- o[16 SG x 128] = As[16 SG x 512] @ W_UV[512 x 128]; wave w owns columns [32w, 32w + 32)
  f32x4 acc[SG][2];
#pragma unroll
  for (int sg = 0; sg < SG; ++sg) acc[sg][0] = acc[sg][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int cc = 0; cc < kWc; ++cc) {
    __syncthreads();
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int e = it * 256 + tid, r = e >> 4, ch = e & 15;
      Ws[16 * r + (ch ^ ws_swz(r))] = wr[cc % AH][it];
    }
    __syncthreads();
    if (cc + AH < kWc) load_chunk(cc + AH);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8 bop[2];
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        // rows 32ks + 8g + j/4 (+4) of the chunk, columns 32w + 16nt + 4(j & 3) .. + 3
        const int c = 4 * w + 2 * nt + ((j & 3) >> 1), r0 = 32 * ks + 8 * g + (j >> 2), r1 = r0 + 4;
        const char* p0 = (const char*)&Ws[16 * r0 + (c ^ ws_swz(r0))] + 8 * (j & 1);
        const char* p1 = (const char*)&Ws[16 * r1 + (c ^ ws_swz(r1))] + 8 * (j & 1);
        const bf16x4 b0v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p0);
        const bf16x4 b1v = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p1);
        bop[nt] = __builtin_shufflevector(b0v, b1v, 0, 1, 2, 3, 4, 5, 6, 7);
      }
#pragma unroll
      for (int sg = 0; sg < SG; ++sg) {
        const int r = 16 * sg + j;
        const bf16x8 a = as_bf16x8(As[r * (kLkv / 8) + ((8 * cc + 4 * ks + g) ^ (r & 15))]);
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) acc[sg][nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bop[nt], acc[sg][nt], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int sg = 0; sg < SG; ++sg)
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int b = b0 + 16 * sg + 4 * g + i;
        if (b < B) out[((size_t)b * kH + h) * kDv + 32 * w + 16 * nt + j] = f32_to_bf16(acc[sg][nt][i]);
      }
}

struct DecodeLayout {
  bf16_t* Qabs;
  int32_t* P;
  int32_t* info;
  bf16_t* zero_row;
  bf16_t* part_o;
  float* part_ml;
  size_t bytes;
};

size_t al(size_t v) { return (v + 255) / 256 * 256; }

DecodeLayout layout(int B, void* base) {
  DecodeLayout L;
  char* p = (char*)base;
  size_t off = 0;
  L.Qabs = (bf16_t*)(p + off);
  off += al((size_t)B * kH * kR * sizeof(bf16_t));
  L.P = (int32_t*)(p + off);
  off += al((size_t)(B + 1) * sizeof(int32_t));
  L.info = (int32_t*)(p + off);
  off += al((size_t)2 * kAttnWGs * sizeof(int32_t));
  L.zero_row = (bf16_t*)(p + off);
  off += al((size_t)kR * sizeof(bf16_t));
  L.part_o = (bf16_t*)(p + off);
  off += al((size_t)(kAttnWGs + B) * kH * kLkv * sizeof(bf16_t));
  L.part_ml = (float*)(p + off);
  off += al((size_t)(kAttnWGs + B) * kH * 2 * sizeof(float));
  L.bytes = off;
  return L;
}

}  // namespace

bool fast_decode_supported(const Dims& d) {
  return d.act == 1 && (d.wk == W_BF16 || d.wk == W_FP8) && d.H == kH && d.Lkv == kLkv && d.dr == kDr &&
         d.dn == kDn && d.dv == kDv && d.bs % kSub == 0;
}

size_t fast_decode_ws_bytes(const Dims& d, int B, int) { return layout(B, nullptr).bytes; }

hipError_t fast_decode_attn(const Dims& d, const void* q, int B, const void* cache, int64_t n_blocks,
                            const int32_t* block_table, int max_blocks, int64_t bt_stride, const int32_t* ctx,
                            const WeightView& wkv_b, void* o, const FastDecodeWs& ws, hipStream_t s) {
  const DecodeLayout L = layout(B, ws.base);
  dim3 fgrid(kH + 1, kLkv / 128, (B + 255) / 256);
  if (d.wk == W_BF16)
    fold_kernel<W_BF16><<<fgrid, 256, 0, s>>>((const bf16_t*)q, B, wkv_b, L.Qabs, ctx, L.P, L.info, L.zero_row);
  else
    fold_kernel<W_FP8><<<fgrid, 256, 0, s>>>((const bf16_t*)q, B, wkv_b, L.Qabs, ctx, L.P, L.info, L.zero_row);
  AttnArgs A;
  A.Qabs = L.Qabs;
  A.cache = (const bf16_t*)cache;
  A.zero_row = L.zero_row;
  A.n_blocks = n_blocks;
  A.bs = d.bs;
  A.bt = block_table;
  A.max_blocks = max_blocks;
  A.bt_stride = bt_stride;
  A.ctx = ctx;
  A.P = L.P;
  A.info = L.info;
  A.B = B;
  A.scale_log2 = d.scale * 1.4426950408889634f;
  A.part_o = L.part_o;
  A.part_ml = L.part_ml;
  decode_attn_kernel<<<kAttnWGs, 64 * kAttnWaves, 0, s>>>(A);
  // 16-sequence groups per combine workgroup (each reusing the head's W_UV chunks already in
  // LDS; the groups' merges run one after another): four for large batches, where W_UV would
  // otherwise be read by B / 16 workgroups per head (B = 256: 48 -> 43 us); one below (at
  // B = 64 two groups per workgroup measured 16.8 us against 15.4)
  const int sg = B >= 256 ? 4 : 1;
  dim3 cgrid(kH, (B + 16 * sg - 1) / (16 * sg));
  auto combine = [&](auto wk, auto sgc) {
    combine_kernel<decltype(wk)::value, decltype(sgc)::value><<<cgrid, 256, 0, s>>>(L.part_o, L.part_ml, L.P, B, wkv_b,
                                                                                  (bf16_t*)o);
  };
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  using WB = std::integral_constant<int, W_BF16>;
  using W8 = std::integral_constant<int, W_FP8>;
  if (d.wk == W_BF16) {
    if (sg == 4) combine(WB{}, I4{});
    else if (sg == 2) combine(WB{}, I2{});
    else combine(WB{}, I1{});
  } else {
    if (sg == 4) combine(W8{}, I4{});
    else if (sg == 2) combine(W8{}, I2{});
    else combine(W8{}, I1{});
  }
  return hipGetLastError();
}

}  // namespace mla
