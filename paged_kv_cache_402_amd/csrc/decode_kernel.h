// Decode attention over a paged KV cache for gfx950 (MI355X).
//
// Pages cited:
//   P1 = openeuler.csdn.net/6ae29ebb40858c2d88170ea6.html (explainer, sections 1-9)
//   P2 = agent.csdn.net/6a744dae662f9a54cb99003e.html (article, sections 1-5)
//   P3 = aiknowledge.cn "2.2 PagedAttention 与 KV Cache 分页管理" (sections 2.2.1-2.2.13)
//
// The operation (P1 §4.2; P3 §2.2.3-§2.2.4): a sequence's keys and values sit in fixed-size
// physical blocks listed by its block table; the kernel reads them block by block through the
// table and computes ordinary softmax attention of the new token's query over all of them.
//
// Work decomposition (our design for gfx950; the pages give no kernel structure):
//   * one 256-lane workgroup (4 waves) per (KV head, context partition of `part` tokens,
//     sequence). Over a host work list (the usual launch) the grid is one-dimensional: row
//     r of the list takes workgroups r * Hkv .. r * Hkv + Hkv - 1, one per KV head; the list
//     holds only partitions that have tokens, full ones first, then the shorter last ones,
//     longest first. Without a list the grid is (Hkv, partitions, sequences). Either way
//     consecutive workgroups differ in KV head and workgroups are dealt to the 8 XCDs
//     round-robin, so with 8 KV heads every workgroup of one head runs on one XCD and blocks
//     shared by many sequences (a common prompt prefix) stay in that XCD's L2;
//   * each wave owns a quarter of the partition and works through it on its own: no
//     workgroup barrier until the final merge, so the four waves never wait for each other
//     and their loads stay in flight independently. A packed row of the work list instead
//     gives each wave a short partition of its own (four items, one KV head), with no merge:
//     a batch of short sequences then needs a quarter of the workgroups;
//   * the partition's physical block ids are loaded once, one per lane, before any KV load;
//     a step's id is then read with v_readlane, so no KV load waits on a table lookup;
//   * K pass: LK lanes (8, or 16 for rows of more than 256 bytes) own one token row; each
//     lane loads 16-byte vectors of it and takes the dot products with its slices of the G
//     query rows of the GQA group (v_dot2 for 16-bit data, held in registers), finished by a
//     DPP butterfly inside the lane group; UK steps of loads are issued before any use. At
//     G = 8 with 16-bit data the scores come from the matrix cores instead (16 tokens x 16
//     padded heads per v_mfma_f32_16x16x32). The scores (in log2 units) go to the wave's own
//     LDS area;
//   * the wave's max, then 2^(s - max) once per (token, head) and the exponent sum; the
//     first round of V loads is issued before this step so it overlaps it;
//   * V pass: LV lanes (16) own one token row; each lane accumulates p * v for its 8 (or 4)
//     columns and every head of the group in fp32;
//   * KV rows are read with the non-temporal cache policy (each row is read once per launch,
//     and on gfx950 such loads read HBM about 12% faster). Every kernel also exists with
//     default-policy KV loads, for launches whose sequences mostly read the same blocks
//     (forks, a long common prefix): there the repeats are served from L2. The caller
//     chooses per launch (kv_policy); the arithmetic is the same;
//   * optional fusions of the decode step: the newest token's K/V rows come from k_new /
//     v_new and are stored into the cache slot; and a copy-on-write of the last block is
//     made by storing the source rows the passes read into the private copy as they are
//     used (only in the kernels built for launches with copy sources, decode_step.hip);
//   * fork groups (the GRP build): the G rows may be several sequences' query heads when
//     those sequences attend to the same tokens before their new one (the branches of a fork
//     right after it, P2 §2.2); the shared tokens are then read once for all of them, and each
//     row's own new token is scored and added by itself after each pass;
//   * the lane rows of a wave are summed with shuffles, then the 4 waves are merged through
//     LDS (each wave's data in its own, now dead, score area) with their maxima; a sequence
//     that fits one partition gets its output row directly, longer ones leave (max, sum,
//     accumulator) partials that a second kernel merges (deterministic split-K, no atomics).
// Tokens past the sequence end, and blocks whose table entry lies outside the pool, are
// excluded by selects and branches, never by multiplying by zero (the slots may hold NaN).
// The arithmetic order does not depend on where blocks sit in the pool.
#pragma once

#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {

template <int DT, int D, int G>
struct Cfg {
  static constexpr int EB = Elem<DT>::bytes;
  static constexpr int PER16 = Elem<DT>::per16;
  static constexpr int RB = D * EB;                    // bytes of one token row of one head
  static constexpr int C = RB / 16;                    // 16-byte vectors per row
  static constexpr int LK = C <= 16 ? 8 : 16;          // lanes per token row, K pass
  static constexpr int NLK = C / LK;                   // vectors per lane per row, K pass
  static constexpr int TK = 64 / LK;                   // token rows per wave step, K pass
  static constexpr int UK = NLK >= 8 ? 1 : 8 / NLK;    // wave steps per load round, K pass
  static constexpr int LV = C < 16 ? C : 16;           // lanes per token row, V pass
  static constexpr int NLV = C / LV;
  static constexpr int TV = 64 / LV;
  static constexpr int UV = NLV >= 8 ? 1 : 8 / NLV;
  static constexpr int ACC = NLV * PER16;              // accumulators per lane per head
  static constexpr int STEP = TK > TV ? TK : TV;       // a wave's share is a multiple of this
  static_assert(C >= 8 && C % LK == 0 && C % LV == 0, "row must be a multiple of 128 bytes");
  static_assert(TK <= 8 && TV <= 8, "a wave step must stay inside one block of >= 8 tokens");
  static_assert(ACC * G <= 64, "accumulators per lane");
};

// Up to 256 block ids per partition, one per lane in 4 registers; j is wave-uniform.
__device__ __forceinline__ int pick_id(const int (&ids)[4], int j) {
  const int sel = j >> 6;
  const int v = sel == 0 ? ids[0] : sel == 1 ? ids[1] : sel == 2 ? ids[2] : ids[3];
  return __builtin_amdgcn_readlane(v, j & 63);
}

// 16x16x32 matrix-core product of 16-bit operands with fp32 accumulation, operands passed as
// the 16 stored bytes each lane holds. Lane l supplies A[l % 16][8 (l / 16) .. +8] and
// B[8 (l / 16) .. +8][l % 16]; it receives C[4 (l / 16) + i][l % 16], i = 0..3.
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
template <int DT> __device__ __forceinline__ f32x4 mfma16x16x32(u32x4 a, u32x4 b, f32x4 c);
template <> __device__ __forceinline__ f32x4 mfma16x16x32<BF16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16x32<F16>(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}
template <> __device__ __forceinline__ f32x4 mfma16x16x32<F32>(u32x4, u32x4, f32x4 c) { return c; }

template <int N> __device__ __forceinline__ void lds_store_n(float* dst, const float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4)
      *reinterpret_cast<float4*>(dst + i) = make_float4(v[i], v[i + 1], v[i + 2], v[i + 3]);
  } else if constexpr (N == 2) {
    *reinterpret_cast<float2*>(dst) = make_float2(v[0], v[1]);
  } else {
    dst[0] = v[0];
  }
}
template <int N> __device__ __forceinline__ void lds_load_n(const float* src, float* v) {
  if constexpr (N % 4 == 0) {
#pragma unroll
    for (int i = 0; i < N; i += 4) {
      const float4 x = *reinterpret_cast<const float4*>(src + i);
      v[i] = x.x; v[i + 1] = x.y; v[i + 2] = x.z; v[i + 3] = x.w;
    }
  } else if constexpr (N == 2) {
    const float2 x = *reinterpret_cast<const float2*>(src);
    v[0] = x.x; v[1] = x.y;
  } else {
    v[0] = src[0];
  }
}

// Work unit of one of the last workgroups of a work-list launch (the last half machine-full):
// the next ticket of the scheduling word, in the list's order. Workgroups are dealt to the
// XCDs round-robin in a fixed share, and XCDs run at slightly different speeds, so a static
// unit per workgroup leaves the fast XCDs idle at the end of the launch; taken this way, the
// units that remain when a workgroup starts go to it, wherever it runs, and the short last
// partitions of the list fill in behind the long ones on every XCD. One atomic per such
// workgroup, no waiting. A word that does not carry the cookie (a workspace that was never
// initialised) leaves every workgroup its static unit.
__device__ __forceinline__ unsigned take_unit(const DecodeArgs& a) {
  const unsigned dyn = (unsigned)(a.work_items * a.num_kv_heads - a.sched_static);
  const unsigned long long old = atomicAdd(a.sched, 1ull);
  const unsigned ticket = (unsigned)old;
  if ((unsigned)(old >> 32) != kSchedCookie || ticket >= dyn) return blockIdx.x;
  if (ticket == dyn - 1) atomicExch(a.sched, (unsigned long long)kSchedCookie << 32);
  return (unsigned)a.sched_static + ticket;
}

// Measurement only: workgroup start and end (s_memrealtime, 100 MHz) and where it ran.
// t_k / t_v: when wave 0 finished its K pass / its V pass (0 where it has none).
__device__ __forceinline__ void record_timeline(const DecodeArgs& a, uint32_t t_start,
                                                unsigned unit, uint32_t t_k, uint32_t t_v,
                                                uint32_t tokens) {
  if (a.timeline != nullptr && threadIdx.x == 0 && blockIdx.x < (unsigned)a.timeline_cap) {
    const uint32_t t_end = (uint32_t)__builtin_amdgcn_s_memrealtime();
    const uint32_t hw_id = __builtin_amdgcn_s_getreg((31 << 11) | 4);     // HW_REG_HW_ID
    const uint32_t xcc_id = __builtin_amdgcn_s_getreg((31 << 11) | 20);   // HW_REG_XCC_ID
    uint32_t* rec = a.timeline + 8 * (size_t)blockIdx.x;
    store16(rec, u32x4{t_start, t_end, hw_id, xcc_id});
    store16(rec + 4, u32x4{unit, t_k, t_v, tokens});
  }
}

__device__ __forceinline__ uint32_t timeline_now(const DecodeArgs& a) {
  return a.timeline != nullptr ? (uint32_t)__builtin_amdgcn_s_memrealtime() : 0u;
}

// NTL: the KV rows are read with the non-temporal cache policy (streaming reads; the default
// choice), else with the default one (batches whose sequences read the same blocks).
// COW: the launch carries copy-on-write sources (cow_src); only those kernels hold the copy's
// stores, so every other launch keeps the registers (and waves per SIMD) it had without them.
// GRP: the work items name fork groups (DecodeArgs::groups) whose members attend to the same
// tokens before their new ones: the group's G rows are several sequences' query heads, the
// shared tokens are read once for all of them, and each row's own new token (its K and V rows
// from k_new / v_new) is scored and added on its own. Launches with k_new and a work list only;
// no matrix-core K pass.
template <int DT, int D, int G, bool MF, bool NTL, bool COW, bool GRP = false>
__global__ __launch_bounds__(kDecodeThreads) void paged_decode_partition_kernel(DecodeArgs a) {
  static_assert(!(GRP && MF), "fork groups take the VALU K pass");
  using K = Cfg<DT, D, G>;
  auto load_kv = [](const unsigned char* p) -> u32x4 {
    if constexpr (NTL) return load16_stream(p);
    else return load16(p);
  };
  constexpr int NW = kDecodeWaves;
  constexpr int NT = kDecodeThreads;
  extern __shared__ __align__(16) unsigned char smem[];
  const uint32_t t_start = a.timeline != nullptr ? (uint32_t)__builtin_amdgcn_s_memrealtime() : 0u;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  int kvh, pi, b;
  unsigned unit = blockIdx.x;   // work unit (list launches: row * Hkv + KV head)
  // packed row: the four waves take four short partitions (four items stored from index
  // idx of the list) of the same KV head, each on its own, with no merge between them
  bool packed = false;
  if (a.work != nullptr) {
    // unit u is (row u / Hkv, KV head u % Hkv): consecutive units take the KV heads of one
    // row, so with 8 KV heads each XCD of the round-robin dispatch keeps to one head for the
    // first resident round (a prefix shared by many sequences stays in that XCD's L2); the
    // last half machine-full of workgroups take their units from the scheduling word when
    // there is one
    if (a.sched != nullptr && (int)blockIdx.x >= a.sched_static) {
      __shared__ unsigned s_unit;
      if (tid == 0) s_unit = take_unit(a);
      __syncthreads();
      unit = s_unit;
    }
    const unsigned item = unit / (unsigned)a.num_kv_heads;
    kvh = unit - item * a.num_kv_heads;
    uint32_t w = a.work[item];
    if (w & kPackedRow) {
      packed = true;
      w = a.work[(w & ~kPackedRow) + wave];
    }
    b = (int)(w >> 16);
    pi = (int)(w & 0xFFFFu);
    if (b >= (GRP ? a.num_groups : a.num_seqs)) return;
  } else {
    kvh = blockIdx.x;
    pi = blockIdx.y;
    b = blockIdx.z;
  }
  // fork group: the sequence of each row (-1: an empty place); its first member's table and
  // length describe the tokens the rows share
  int rowseq[G];
  int lead = b;
  if constexpr (GRP) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int m = a.groups[(size_t)b * a.group_size + g / a.group_heads];
      rowseq[g] = (unsigned)m < (unsigned)a.num_seqs ? m : -1;
    }
    lead = rowseq[0];
    if (lead < 0) return;
  }
  const int t0 = pi * a.part;                  // a multiple of the block size
  // ---- block ids of the partition (one per lane) and the query slices, issued together with
  // the length load: every table entry the partition could use (those past the sequence end
  // are never read again), so no load waits on another before the first K round ----
  const int32_t* __restrict__ trow =
      a.block_tables + (size_t)lead * a.max_blocks + (t0 >> a.bs_log2);
  const int pblk = min(a.part >> a.bs_log2, a.max_blocks - (t0 >> a.bs_log2));
  int ids[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int j = k * 64 + lane;
    ids[k] = j < pblk ? trow[j] : 0;
  }
  const int kr = lane / K::LK;  // token row inside a K step
  const int kc = lane % K::LK;  // this lane's vectors: kc, kc+LK, ...
  const unsigned char* qsrc =
      (const unsigned char*)a.q + ((size_t)b * a.num_q_heads + (size_t)kvh * G) * K::RB;
  // query row of row g: head kvh * G + g of sequence b, or of a fork group's member
  auto qrow = [&](int g) -> const unsigned char* {
    if constexpr (GRP)
      return (const unsigned char*)a.q +
             ((size_t)max(rowseq[g], 0) * a.num_q_heads + (size_t)kvh * a.group_heads +
              g % a.group_heads) * K::RB;
    else
      return qsrc + (size_t)g * K::RB;
  };
  u32x4 qv[G][K::NLK];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int i = 0; i < K::NLK; ++i)
      qv[g][i] = load16(qrow(g) + (size_t)(kc + i * K::LK) * 16);
  // fork group with few enough rows (HOIST): each row's own new token costs no round trip of
  // its own. Its K row (k_new; the address needs only the member) is loaded beside the query
  // slices and scored before the K pass; its V row is loaded with the first V round. The rows'
  // new K and V rows for their cache slots are spread over the lanes of one wave (wave 0, or
  // each wave of a packed row, which has a group of its own), loaded here and stored once the K
  // pass is done. More rows, or fp32 rows, would take registers enough to cost a wave per
  // SIMD: they load their own rows after each pass instead.
  constexpr bool HOIST = GRP && DT != F32 && G <= 4 && G * K::NLK <= 8;
  constexpr int OWN_PER_LANE = (2 * G * K::C + 63) / 64;    // 16-byte pieces, K rows then V
  u32x4 kown[HOIST ? G : 1][K::NLK];
  u32x4 own_put[HOIST ? OWN_PER_LANE : 1];
  // row g's new K or V row (g known at compile time: the register arrays are never indexed
  // at run time, which would send them to scratch memory)
  auto own_row = [&](int g, bool isv) -> const unsigned char* {
    const unsigned char* base = (const unsigned char*)(isv ? a.v_new : a.k_new);
    return base + ((size_t)max(rowseq[g], 0) * a.num_kv_heads + kvh) * K::RB;
  };
  // piece j of this lane in the spread of the 2G own rows: row j * RPP + lane / C of them
  // (the K rows, then the V rows), column lane % C
  constexpr int RPP = 64 / K::C;                             // rows per pass of the lanes
  const bool own_wave = packed || wave == 0;                 // the wave that stores them
  // (a fork-group launch always carries k_new and v_new; the test keeps a launch without
  // them from reading through null)
  if constexpr (HOIST) if (a.k_new != nullptr && a.v_new != nullptr) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < K::NLK; ++i)
        kown[g][i] = load16(own_row(g, false) + (size_t)(kc + i * K::LK) * 16);
#pragma unroll
    for (int j = 0; j < OWN_PER_LANE; ++j) {
      own_put[j] = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) {
        const int r = j * RPP + rr;
        if (own_wave && r < 2 * G && lane / K::C == rr)
          own_put[j] = load16(own_row(r % G, r >= G) + (size_t)(lane % K::C) * 16);
      }
    }
  }
  const int cap = a.max_blocks << a.bs_log2;
  int L = a.seq_lens[lead];
  L = L < 0 ? 0 : (L > cap ? cap : L);
  const int nparts = L == 0 ? 1 : (L + a.part - 1) / a.part;
  if (pi >= nparts) return;
  const int n = max(0, min(L - t0, a.part));   // tokens of this partition
  // a packed wave's partition must fit its LDS area (the list builder packs at most
  // part / 4 tokens); a list that breaks this leaves the item unwritten
  if (packed && n > a.part / NW) return;

  // this wave's share of the partition: [c0, c0 + nw), partition-relative; a multiple of
  // every step size (the matrix-core K pass takes 16 tokens per step). A packed wave takes
  // its whole partition.
  constexpr int STEP = MF && K::STEP < 16 ? 16 : K::STEP;
  const int share = (((n + NW - 1) / NW) + STEP - 1) / STEP * STEP;
  const int c0 = packed ? 0 : min(n, wave * share);
  const int nw = packed ? n : min(n - c0, share);

  // LDS: one area per wave, [part/NW][G] scores; after its V pass the wave's scores are dead
  // and its merge data ([G][D] accumulator, [G] max, [G] sum) go in their place, so the
  // workgroup needs no separate merge area (at 2048-token partitions and G = 4 that keeps it
  // at 32 KiB, five workgroups' worth of a compute unit's 160 KiB instead of three)
  const int wstride = max(a.part / NW, D + 2) * G;      // floats per wave
  float* s_sc = reinterpret_cast<float*>(smem) + (size_t)wave * wstride;
  auto w_acc = [&](int w) { return reinterpret_cast<float*>(smem) + (size_t)w * wstride; };
  auto w_m = [&](int w) { return w_acc(w) + G * D; };
  auto w_l = [&](int w) { return w_acc(w) + G * D + G; };

  const int bs_mask = (1 << a.bs_log2) - 1;
  const size_t head_bytes = ((size_t)1 << a.bs_log2) * K::RB;   // one (block, head) tile
  const size_t block_bytes = head_bytes * a.num_kv_heads;       // one block, all heads
  const unsigned char* kbase = (const unsigned char*)a.k_cache + kvh * head_bytes;
  const unsigned char* vbase = (const unsigned char*)a.v_cache + kvh * head_bytes;

  // ---- appended token (optional): the K and V rows of token L - 1 come from k_new /
  // v_new instead of the cache, and the workgroup of (KV head, last partition) stores them
  // into the cache slot the table gives; no other workgroup reads that slot in this launch
  const bool fused = a.k_new != nullptr;
  const int last = L - 1 - t0;                       // partition-relative; outside [0, n): none
  const size_t new_off = ((size_t)b * a.num_kv_heads + kvh) * K::RB;
  const unsigned char* knew = fused ? (const unsigned char*)a.k_new + new_off : nullptr;
  const unsigned char* vnew = fused ? (const unsigned char*)a.v_new + new_off : nullptr;
  // copy-on-write of the last block (optional): the block the sequence shared until this
  // step's append. The passes read the earlier tokens of the last block from it, and every
  // lane that loads one of those rows (of this KV head) also stores it into the new private
  // block when it uses it, so the copy costs stores only and no phase of its own. The new
  // token's row is written by the store below; rows past it hold no token of the sequence
  // and are left as they are (an append writes them before any read).
  const int cow = (COW && fused && a.cow_src != nullptr && last >= 0 && last < n) ? a.cow_src[lead] : -1;
  const int cow_dst =
      (unsigned)cow < (unsigned)a.num_blocks ? pick_id(ids, last >> a.bs_log2) : -1;
  const bool cow_live = (unsigned)cow < (unsigned)a.num_blocks && (unsigned)cow_dst < (unsigned)a.num_blocks;
  // fork group, per row g: the block of its member's table that holds the new token (-1:
  // none), and the same block as a copy destination when the member made a private copy of it
  // (only on the first row of each member, so each copy is stored once); the loads of all rows
  // are independent and issue together
  int rblk[G], gdst[G];
  bool any_gdst = false;
  if constexpr (GRP) {
    const bool here = fused && last >= 0 && last < n;
    const size_t jabs = (size_t)(t0 >> a.bs_log2) + (size_t)(max(last, 0) >> a.bs_log2);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const int blk =
          here && rowseq[g] >= 0 ? a.block_tables[(size_t)rowseq[g] * a.max_blocks + jabs] : -1;
      rblk[g] = (unsigned)blk < (unsigned)a.num_blocks ? blk : -1;
      const int src = COW && here && rowseq[g] >= 0 && g % a.group_heads == 0 &&
                              a.cow_src != nullptr ? a.cow_src[rowseq[g]] : -1;
      gdst[g] = (unsigned)src < (unsigned)a.num_blocks ? rblk[g] : -1;
      any_gdst |= gdst[g] >= 0;
    }
  }
  const int cow_jb = (GRP ? any_gdst : cow_live) ? last >> a.bs_log2 : -1;   // the last block, partition-relative
  // this KV head's tiles of the private copy (uniform; cow_live has checked the block id, and
  // every store below lands inside the tile: row < block_size, column < the row's bytes)
  unsigned char* const cow_k =
      const_cast<unsigned char*>(kbase) + (size_t)(cow_live ? cow_dst : 0) * block_bytes;
  unsigned char* const cow_v =
      const_cast<unsigned char*>(vbase) + (size_t)(cow_live ? cow_dst : 0) * block_bytes;
  // one 16-byte piece of a copied row (off: its byte offset in the tile) into the copy, or
  // into every member's copy of a fork group
  auto cow_put = [&](const unsigned char* base, unsigned char* one, size_t off, const u32x4& v) {
    if constexpr (GRP) {
#pragma unroll
      for (int j = 0; j < G; ++j)
        if (gdst[j] >= 0)
          store16(const_cast<unsigned char*>(base) + (size_t)gdst[j] * block_bytes + off, v);
    } else {
      store16(one + off, v);
    }
  };
  if (!GRP && fused && last >= 0 && last < n && (packed || wave == 0)) {
    const int blk = pick_id(ids, last >> a.bs_log2);
    if ((unsigned)blk < (unsigned)a.num_blocks) {
      const size_t row = (size_t)blk * block_bytes + (size_t)(last & bs_mask) * K::RB;
      for (int c = lane; c < 2 * K::C; c += 64) {
        const bool isv = c >= K::C;
        const int cc = isv ? c - K::C : c;
        unsigned char* dst = (unsigned char*)(isv ? a.v_cache : a.k_cache) + kvh * head_bytes + row;
        store16(dst + cc * 16, load16((isv ? vnew : knew) + cc * 16));
      }
    }
  }
  if ((unsigned)cow < (unsigned)a.num_blocks) {
    // every wave of the partition reads the last block's earlier tokens from the source
    const int jb = last >> a.bs_log2;
#pragma unroll
    for (int k = 0; k < 4; ++k)
      if (k == (jb >> 6) && lane == (jb & 63)) ids[k] = cow;
  }


  // fork group (HOIST): each row's own score, from the K row loaded with the query slices
  float so[HOIST ? G : 1];
  if constexpr (HOIST) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float acc = 0.f;
#pragma unroll
      for (int i = 0; i < K::NLK; ++i) acc = dot16<DT>(qv[g][i], kown[g][i], acc);
      so[g] = rowseq[g] >= 0 ? group_sum<K::LK>(acc) * a.scale_log2 : -INFINITY;
    }
  }

  // ---- K pass over the wave's share: scores (log2 units) -> LDS, running max ----
  float m[G];
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = -INFINITY;
  if constexpr (MF) {
    // Matrix cores: S^T (16 padded heads x 16 tokens) = Q (16 x d) . K^T (d x 16), d in
    // slices of 32. Lane l holds head / token l % 16 and the 8 elements 32 j + 8 (l / 16) of
    // slice j; the result gives lane l the scores of token l % 16 for heads 4 (l / 16) + i.
    constexpr int NJ = D / 32;                    // products per 16-token step
    constexpr int UM = NJ >= 8 ? 1 : 8 / NJ;      // steps per load round (8 loads per lane)
    const int rl = lane & 15;
    const int kg = lane >> 4;
    u32x4 qa[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j)
      qa[j] = rl < G ? load16(qsrc + (size_t)rl * K::RB + j * 64 + kg * 16) : u32x4{0u, 0u, 0u, 0u};
    float mh[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) mh[i] = -INFINITY;
    const int ngm = (nw + 15) / 16;
    for (int g0 = 0; g0 < ngm; g0 += UM) {
      u32x4 kb[UM][NJ];
      bool okb[UM];
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int gi = g0 + u;
        okb[u] = false;
        if (gi < ngm) {
          const int tok = c0 + gi * 16;
          const int blk = pick_id(ids, tok >> a.bs_log2);
          okb[u] = (unsigned)blk < (unsigned)a.num_blocks;
          const unsigned char* p = kbase + (size_t)(okb[u] ? blk : 0) * block_bytes +
                                   (uint32_t)(((tok & bs_mask) + rl) * K::RB + kg * 16);
          if (fused && tok + rl == last) p = knew + kg * 16;
#pragma unroll
          for (int j = 0; j < NJ; ++j) kb[u][j] = load_kv(p + j * 64);
        } else {
#pragma unroll
          for (int j = 0; j < NJ; ++j) kb[u][j] = u32x4{0u, 0u, 0u, 0u};
        }
      }
#pragma unroll
      for (int u = 0; u < UM; ++u) {
        const int gi = g0 + u;
        if (gi < ngm) {
          const int tl = gi * 16 + rl;
          const int tok = c0 + gi * 16;
          if (COW && (tok >> a.bs_log2) == cow_jb && tok + rl < last && tl < nw) {
#pragma unroll
            for (int j = 0; j < NJ; ++j)
              store16(cow_k + ((tok & bs_mask) + rl) * K::RB + kg * 16 + j * 64, kb[u][j]);
          }
          f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int j = 0; j < NJ; ++j) c = mfma16x16x32<DT>(qa[j], kb[u][j], c);
          const bool valid = okb[u] && tl < nw;
          float sv[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            sv[i] = valid ? c[i] * a.scale_log2 : -INFINITY;
            mh[i] = fmaxf(mh[i], sv[i]);
          }
          if (tl < nw && kg * 4 < G) lds_store_n<(G < 4 ? G : 4)>(s_sc + tl * G + kg * 4, sv);
        }
      }
    }
    // max over the 16 tokens of each lane row, then broadcast head g from row g / 4
#pragma unroll
    for (int i = 0; i < 4; ++i) mh[i] = xor_max_row16(mh[i]);
#pragma unroll
    for (int g = 0; g < G; ++g)
      m[g] = __builtin_bit_cast(float, __builtin_amdgcn_readlane(
                                           __builtin_bit_cast(int, mh[g & 3]), (g >> 2) * 16));
  } else {
  const int ngk = (nw + K::TK - 1) / K::TK;
  for (int g0 = 0; g0 < ngk; g0 += K::UK) {
    u32x4 kv[K::UK][K::NLK];
    bool okb[K::UK];
#pragma unroll
    for (int u = 0; u < K::UK; ++u) {
      const int gi = g0 + u;
      okb[u] = false;
      if (gi < ngk) {
        const int tok = c0 + gi * K::TK;
        const int blk = pick_id(ids, tok >> a.bs_log2);
        okb[u] = (unsigned)blk < (unsigned)a.num_blocks;
        const unsigned char* p = kbase + (size_t)(okb[u] ? blk : 0) * block_bytes +
                                 (uint32_t)(((tok & bs_mask) + kr) * K::RB + kc * 16);
        if (!GRP && fused && tok + kr == last) p = knew + kc * 16;
#pragma unroll
        for (int i = 0; i < K::NLK; ++i) kv[u][i] = load_kv(p + i * K::LK * 16);
      } else {
#pragma unroll
        for (int i = 0; i < K::NLK; ++i) kv[u][i] = u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int u = 0; u < K::UK; ++u) {
      const int gi = g0 + u;
      if (gi < ngk) {
        const int tl = gi * K::TK + kr;
        const int tok = c0 + gi * K::TK;
        if (COW && (tok >> a.bs_log2) == cow_jb && tok + kr < last && tl < nw) {
#pragma unroll
          for (int i = 0; i < K::NLK; ++i)
            cow_put(kbase, cow_k, (size_t)((tok & bs_mask) + kr) * K::RB + (kc + i * K::LK) * 16,
                    kv[u][i]);
        }
        float s[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
          float acc = 0.f;
#pragma unroll
          for (int i = 0; i < K::NLK; ++i) acc = dot16<DT>(qv[g][i], kv[u][i], acc);
          s[g] = group_sum<K::LK>(acc) * a.scale_log2;
        }
        // a fork group's rows each have their own new token: scored after the pass
        const bool valid = okb[u] && tl < nw && !(GRP && tok + kr == last);
#pragma unroll
        for (int g = 0; g < G; ++g) {
          s[g] = valid ? s[g] : -INFINITY;
          m[g] = fmaxf(m[g], s[g]);
        }
        if (kc == 0 && tl < nw) lds_store_n<G>(s_sc + tl * G, s);
      }
    }
  }
  if constexpr (HOIST) {
    // each row's own score into the slot of its new token (the pass above left -inf there)
    if (fused && last >= c0 && last < c0 + nw) {
#pragma unroll
      for (int g = 0; g < G; ++g) m[g] = fmaxf(m[g], so[g]);
      if (lane == 0) lds_store_n<G>(s_sc + (last - c0) * G, so);
    }
    // the members' new K and V rows into their cache slots: a member's first row only, so
    // each is stored once (rblk: -1 unless this partition holds the new token)
#pragma unroll
    for (int j = 0; j < OWN_PER_LANE; ++j)
#pragma unroll
      for (int rr = 0; rr < RPP; ++rr) {
        const int r = j * RPP + rr;
        if (own_wave && r < 2 * G && lane / K::C == rr && rblk[r % G] >= 0 &&
            (r % G) % a.group_heads == 0) {
          unsigned char* slot = (unsigned char*)(r >= G ? a.v_cache : a.k_cache) +
                                kvh * head_bytes + (size_t)rblk[r % G] * block_bytes +
                                (size_t)(last & bs_mask) * K::RB;
          store16(slot + (size_t)(lane % K::C) * 16, own_put[j]);
        }
      }
  } else if constexpr (GRP) {
    // each row's own new token: its score against the member's K row from k_new, into the
    // slot of that position (the pass above left -inf there)
    if (fused && last >= c0 && last < c0 + nw) {
      float so[G];
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const unsigned char* kn = (const unsigned char*)a.k_new +
                                  ((size_t)max(rowseq[g], 0) * a.num_kv_heads + kvh) * K::RB;
        // the member's new K row also goes into its cache slot (once per member: its first
        // row, by the lanes of the first token row)
        unsigned char* slot = (unsigned char*)a.k_cache + kvh * head_bytes +
                              (size_t)max(rblk[g], 0) * block_bytes +
                              (size_t)(last & bs_mask) * K::RB;
        const bool put = kr == 0 && rblk[g] >= 0 && g % a.group_heads == 0;
        float acc = 0.f;
#pragma unroll
        for (int i = 0; i < K::NLK; ++i) {
          const u32x4 kx = load16(kn + (kc + i * K::LK) * 16);
          if (put) store16(slot + (kc + i * K::LK) * 16, kx);
          acc = dot16<DT>(qv[g][i], kx, acc);
        }
        so[g] = rowseq[g] >= 0 ? group_sum<K::LK>(acc) * a.scale_log2 : -INFINITY;
        m[g] = fmaxf(m[g], so[g]);
      }
      if (lane == 0) lds_store_n<G>(s_sc + (last - c0) * G, so);
    }
  }
  // the wave's max (every lane ends with it); -inf when the share has no readable token
#pragma unroll
  for (int g = 0; g < G; ++g) m[g] = xor_max_from<K::LK>(m[g]);
  }

  const uint32_t t_k = timeline_now(a);

  // ---- first round of V loads, issued before the exponentials ----
  const int vr = lane / K::LV;
  const int vc = lane % K::LV;
  const int ngv = (nw + K::TV - 1) / K::TV;
  u32x4 vv[K::UV][K::NLV];
  bool okv[K::UV];
  auto load_v = [&](int g0) {
#pragma unroll
    for (int u = 0; u < K::UV; ++u) {
      const int gi = g0 + u;
      okv[u] = false;
      if (gi < ngv) {
        const int tok = c0 + gi * K::TV;
        const int blk = pick_id(ids, tok >> a.bs_log2);
        okv[u] = (unsigned)blk < (unsigned)a.num_blocks;
        const unsigned char* p = vbase + (size_t)(okv[u] ? blk : 0) * block_bytes +
                                 (uint32_t)(((tok & bs_mask) + vr) * K::RB + vc * 16);
        if (!GRP && fused && tok + vr == last) p = vnew + vc * 16;
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) vv[u][i] = load_kv(p + i * K::LV * 16);
      }
    }
  };
  // fork group (HOIST): the own rows' V rows, loaded with the first V round by the lanes that
  // add them (the first row group of the wave that holds the new token)
  const bool own_v = HOIST && fused && last >= c0 && last < c0 + nw && vr == 0;
  u32x4 vown[HOIST ? G : 1][K::NLV];
  if constexpr (HOIST) {
    if (own_v) {
#pragma unroll
      for (int g = 0; g < G; ++g)
#pragma unroll
        for (int i = 0; i < K::NLV; ++i)
          vown[g][i] = load16(own_row(g, true) + (size_t)(vc + i * K::LV) * 16);
    }
  }
  load_v(0);

  // ---- probabilities 2^(s - max) in place, once per (token, head); their sum ----
  float l[G];
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = 0.f;
  __builtin_amdgcn_wave_barrier();
  float mz[G];  // exponent base: the max, or 0 when nothing is readable (then every p is 0)
#pragma unroll
  for (int g = 0; g < G; ++g) mz[g] = m[g] == -INFINITY ? 0.f : m[g];
  for (int t = lane; t < nw; t += 64) {
    float v[G];
    lds_load_n<G>(s_sc + t * G, v);
#pragma unroll
    for (int g = 0; g < G; ++g) {
      v[g] = exp2f(v[g] - mz[g]);  // a stored -inf gives 0
      l[g] += v[g];
    }
    lds_store_n<G>(s_sc + t * G, v);
  }
#pragma unroll
  for (int g = 0; g < G; ++g) l[g] = xor_sum_from<1>(l[g]);
  __builtin_amdgcn_wave_barrier();

  // ---- V pass: acc[g][:] += p[g] * v over the wave's share ----
  float acc[G][K::ACC];
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < K::ACC; ++e) acc[g][e] = 0.f;
  if constexpr (HOIST) {
    // each row's own new token first: its weight times the member's V row
    if (own_v) {
      float pg[G];
      lds_load_n<G>(s_sc + (last - c0) * G, pg);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (rowseq[g] < 0) continue;
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) {
          float f[K::PER16];
          widen<DT>(vown[g][i], f);
#pragma unroll
          for (int e = 0; e < K::PER16; ++e)
            acc[g][i * K::PER16 + e] = __builtin_fmaf(pg[g], f[e], acc[g][i * K::PER16 + e]);
        }
      }
    }
  }
  for (int g0 = 0; g0 < ngv; g0 += K::UV) {
    if (g0 > 0) load_v(g0);
#pragma unroll
    for (int u = 0; u < K::UV; ++u) {
      const int gi = g0 + u;
      const int tl = gi * K::TV + vr;
      const int tok = c0 + gi * K::TV;
      if (COW && gi < ngv && (tok >> a.bs_log2) == cow_jb && tok + vr < last && tl < nw) {
#pragma unroll
        for (int i = 0; i < K::NLV; ++i)
          cow_put(vbase, cow_v, (size_t)((tok & bs_mask) + vr) * K::RB + (vc + i * K::LV) * 16,
                  vv[u][i]);
      }
      // tokens past the sequence end may hold anything (even NaN): skip, never multiply by 0
      if (gi < ngv && okv[u] && tl < nw && !(GRP && tok + vr == last)) {
        float pg[G];
        lds_load_n<G>(s_sc + tl * G, pg);
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) {
          float f[K::PER16];
          widen<DT>(vv[u][i], f);
#pragma unroll
          for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < K::PER16; ++e)
              acc[g][i * K::PER16 + e] = __builtin_fmaf(pg[g], f[e], acc[g][i * K::PER16 + e]);
        }
      }
    }
  }

  if constexpr (GRP && !HOIST) {
    // each row's own new token: its weight times the member's V row from v_new, once per
    // column (the lanes of the first row group)
    if (fused && last >= c0 && last < c0 + nw && vr == 0) {
      float pg[G];
      lds_load_n<G>(s_sc + (last - c0) * G, pg);
#pragma unroll
      for (int g = 0; g < G; ++g) {
        if (rowseq[g] < 0) continue;
        const unsigned char* vn = (const unsigned char*)a.v_new +
                                  ((size_t)rowseq[g] * a.num_kv_heads + kvh) * K::RB;
        // the member's new V row also goes into its cache slot (once per member)
        unsigned char* slot = (unsigned char*)a.v_cache + kvh * head_bytes +
                              (size_t)max(rblk[g], 0) * block_bytes +
                              (size_t)(last & bs_mask) * K::RB;
        const bool put = rblk[g] >= 0 && g % a.group_heads == 0;
#pragma unroll
        for (int i = 0; i < K::NLV; ++i) {
          const u32x4 vx = load16(vn + (vc + i * K::LV) * 16);
          if (put) store16(slot + (vc + i * K::LV) * 16, vx);
          float f[K::PER16];
          widen<DT>(vx, f);
#pragma unroll
          for (int e = 0; e < K::PER16; ++e)
            acc[g][i * K::PER16 + e] = __builtin_fmaf(pg[g], f[e], acc[g][i * K::PER16 + e]);
        }
      }
    }
  }

  const uint32_t t_v = timeline_now(a);

  // ---- the wave's rows summed; the wave's (max, sum, accumulator) -> LDS ----
#pragma unroll
  for (int g = 0; g < G; ++g)
#pragma unroll
    for (int e = 0; e < K::ACC; ++e) acc[g][e] = xor_sum_from<K::LV>(acc[g][e]);

  const bool single = nparts == 1;
  if (packed) {
    // the merge of one wave: f = 1 (0 when nothing was readable), out = acc / l
    if (vr == 0) {
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int sq = GRP ? rowseq[g] : b;                 // the row's sequence
        if (sq < 0) continue;
        const int h = GRP ? kvh * a.group_heads + g % a.group_heads : kvh * G + g;
        const float f = m[g] == -INFINITY ? 0.f : 1.f;
        const float den = __builtin_fmaf(f, l[g], 0.f);
        const size_t slot = ((size_t)sq * a.num_q_heads + h) * a.pmax + pi;
#pragma unroll
        for (int i = 0; i < K::NLV; ++i)
#pragma unroll
          for (int e = 0; e < K::PER16; ++e) {
            const int d = (i * K::LV + vc) * K::PER16 + e;
            const float num = __builtin_fmaf(f, acc[g][i * K::PER16 + e], 0.f);
            if (single)
              store_out(a.out, ((size_t)sq * a.num_q_heads + h) * D + d,
                        den > 0.f ? num / den : 0.f, a.out_dtype);
            else
              a.ws_acc[slot * D + d] = num;
          }
        if (!single && vc == 0) {
          a.ws_ml[slot * 2] = m[g];
          a.ws_ml[slot * 2 + 1] = den;
        }
      }
    }
    record_timeline(a, t_start, unit, t_k, t_v, (uint32_t)n);
    return;
  }
  // every lane's score reads are done before the area is reused (LDS keeps a wave's order)
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
  if (vr == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
      for (int i = 0; i < K::NLV; ++i)
        lds_store_n<K::PER16>(w_acc(wave) + g * D + (i * K::LV + vc) * K::PER16,
                              &acc[g][i * K::PER16]);
  }
  if (lane == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      w_m(wave)[g] = m[g];
      w_l(wave)[g] = l[g];
    }
  }
  __syncthreads();

  // ---- merge the waves; write the output row or this partition's partials ----
  for (int idx = tid; idx < G * D; idx += NT) {
    const int g = idx / D;
    const int d = idx - g * D;
    float M = w_m(0)[g];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, w_m(w)[g]);
    float num = 0.f, den = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float mw = w_m(w)[g];
      const float f = mw == -INFINITY ? 0.f : exp2f(mw - M);
      num = __builtin_fmaf(f, w_acc(w)[g * D + d], num);
      den = __builtin_fmaf(f, w_l(w)[g], den);
    }
    int sq = b;                                              // the row's sequence
    if constexpr (GRP) {
      const int mm = a.groups[(size_t)b * a.group_size + g / a.group_heads];
      sq = (unsigned)mm < (unsigned)a.num_seqs ? mm : -1;
    }
    if (sq < 0) continue;
    const int h = GRP ? kvh * a.group_heads + g % a.group_heads : kvh * G + g;
    if (single) {
      const float y = den > 0.f ? num / den : 0.f;
      store_out(a.out, ((size_t)sq * a.num_q_heads + h) * D + d, y, a.out_dtype);
    } else {
      const size_t slot = ((size_t)sq * a.num_q_heads + h) * a.pmax + pi;
      a.ws_acc[slot * D + d] = num;
      if (d == 0) {
        a.ws_ml[slot * 2] = M;  // -inf when the partition had no readable token
        a.ws_ml[slot * 2 + 1] = den;
      }
    }
  }
  record_timeline(a, t_start, unit, t_k, t_v, (uint32_t)n);
}

// Workgroups of `kernel` resident at once on the current device with `lds` bytes of dynamic
// LDS (occupancy query, cached per kernel, LDS size and device); 0 if unknown.
int resident_groups(const void* kernel, size_t lds);

// The first unit of a work-list launch of `units` units that is handed out by ticket (units:
// none), for a kernel of which `resident` workgroups fit on the device at once (0: unknown).
// Only the last half machine-full of units (half as many as fit at once) is handed out by
// ticket: the list runs longest first, so those are its shortest units, enough to even out
// the XCDs' finishing times. Every earlier workgroup keeps its static unit, and with it the
// XCD of its KV head: a unit moved to another XCD reads the blocks its sequences share (a
// common prefix) from HBM again instead of that XCD's L2. With non-temporal KV loads,
// ticketing a whole machine-full cost more in such re-reads than it saved.
static inline int ticket_start(int units, int resident) {
  const int late = resident / 2;
  const int first = units - late > resident ? units - late : resident;
  return late <= 0 || first >= units ? units : first;
}

// With `ticketed` non-null nothing is launched: *ticketed receives how many of the launch's
// units would be handed out by ticket (an error if the occupancy query fails).
template <int DT, int D, int G, bool MF, bool NTL, bool COW, bool GRP = false>
static hipError_t launch_k(DecodeArgs a, size_t lds, hipStream_t stream, int* ticketed) {
  const auto kernel = paged_decode_partition_kernel<DT, D, G, MF, NTL, COW, GRP>;
  if (ticketed != nullptr) {
    const int units = a.num_kv_heads * a.work_items;
    const int resident = resident_groups((const void*)kernel, lds);
    if (resident <= 0) return hipErrorNoDevice;
    *ticketed = units - ticket_start(units, resident);
    return hipSuccess;
  }
  if (a.work != nullptr) {
    const int units = a.num_kv_heads * a.work_items;
    const int resident = a.sched != nullptr ? resident_groups((const void*)kernel, lds) : 0;
    a.sched_static = ticket_start(units, resident);
    if (a.sched_static >= units) a.sched = nullptr;
    hipLaunchKernelGGL(kernel, dim3((unsigned)units), dim3(kDecodeThreads), lds, stream, a);
  } else {
    a.sched = nullptr;
    hipLaunchKernelGGL(kernel, dim3(a.num_kv_heads, a.pmax, a.num_seqs), dim3(kDecodeThreads),
                       lds, stream, a);
  }
  return hipGetLastError();
}

template <int DT, int D, int G, bool COW, bool GRP = false>
static hipError_t launch_t(const DecodeArgs& a, hipStream_t stream, int* ticketed) {
  const size_t lds = decode_lds_bytes(DT, D, G, a.part);
  // Matrix-core scores for 16-bit data at G = 8, when a 16-token step stays inside one block
  // and the waves' shares (part / 4) are whole steps. At G <= 4 the VALU dot products measured
  // faster (the padded 16-row product does 4x the work there and the K pass is not the limit).
  // Fork groups take the VALU pass.
  constexpr bool kMF = DT != F32 && G == 8 && !GRP;
  const bool mf = kMF && a.bs_log2 >= 4 && a.part % 64 == 0;
  if (a.kv_cached)
    return mf ? launch_k<DT, D, G, kMF, false, COW, GRP>(a, lds, stream, ticketed)
              : launch_k<DT, D, G, false, false, COW, GRP>(a, lds, stream, ticketed);
  return mf ? launch_k<DT, D, G, kMF, true, COW, GRP>(a, lds, stream, ticketed)
            : launch_k<DT, D, G, false, true, COW, GRP>(a, lds, stream, ticketed);
}

// group: the rows of a workgroup (query heads per KV head, times the members of a fork group)
template <int DT, int D, bool COW, bool GRP = false>
static hipError_t launch_g(const DecodeArgs& a, int group, hipStream_t stream,
                            int* ticketed) {
  switch (group) {
    case 1: return launch_t<DT, D, 1, COW, GRP>(a, stream, ticketed);
    case 2: return launch_t<DT, D, 2, COW, GRP>(a, stream, ticketed);
    case 4: return launch_t<DT, D, 4, COW, GRP>(a, stream, ticketed);
    case 8:
      if constexpr (D <= 128) return launch_t<DT, D, 8, COW, GRP>(a, stream, ticketed);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

template <int DT, bool COW, bool GRP = false>
static hipError_t launch_d(const DecodeArgs& a, int head_dim, int group, hipStream_t stream,
                            int* ticketed) {
  switch (head_dim) {
    case 64: return launch_g<DT, 64, COW, GRP>(a, group, stream, ticketed);
    case 128: return launch_g<DT, 128, COW, GRP>(a, group, stream, ticketed);
    case 256: return launch_g<DT, 256, COW, GRP>(a, group, stream, ticketed);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pkv

