// Exact-attention backward for AMD CDNA4 (gfx950, MI355X), and its C ABI.
//
// What it computes (FlashAttention-4 (papercache summary), section 2.1, the
// backward equations): for S = scale Q K^T (masked), P = softmax(S), O = P V
// and an upstream gradient dO,
//     dV = P^T dO,  dP = dO V^T,  dS = P * (dP - D)  (D_i = <dO_i, O_i>),
//     dQ = scale dS K,  dK = scale dS^T Q,
// with P rebuilt from the forward's saved LSE as exp(S - LSE), so no N x N
// matrix is stored ("059 · FlashAttention" (wq-win), section 3: the backward
// recomputes probability blocks from the inputs and the saved row
// statistics).  Grouped-query heads: a KV head's gradient sums its G query
// heads.
//
// Three kernels, no atomics, deterministic:
// * bwd_preprocess: D = <dO, O> per row, and LSE in log2 units (+inf for a
//   row with no visible key, so exp2(s - lse) is 0 there), into a workspace.
// * bwd_dkdv_pp_kernel: one workgroup of 8 waves per 128 keys of one (batch,
//   KV head).  Waves w and w+4 own keys 32(w%4)..+31 and share a SIMD; the two
//   groups take alternate query steps (32 rows of one of the G query heads)
//   and alternate MFMA and VALU phases half a period apart.  S = Q K^T is
//   formed with the keys as the columns of the 32x32 MFMA accumulator, so
//   each lane holds one key and 16 queries: P and dS are then B operands
//   (k = queries) of dV^T += dO^T P and dK^T += Q^T dS without leaving
//   registers; dO^T and Q^T come from gfx950 transpose reads of LDS
//   (ds_read_b64_tr_b16).  The groups' partial sums are added through LDS
//   in a fixed order.  The recompute ordering of FlashAttention-4
//   (papercache summary), section 3.2.2: iterate along the KV sequence,
//   values transposed relative to the forward.
// * bwd_dq_pp_kernel: one workgroup of 8 waves per 256 query rows of one
//   head (or 256 / P rows of each of P query heads of one KV group), the
//   forward's orientation (S^T = K Q^T, one query per lane), with
//   dP^T = V dO^T, dS^T = P^T * (dP^T - D) and dQ^T += K^T dS^T over key
//   tiles of 32.  The two wave groups alternate MFMA and VALU phases half a
//   period apart, as the forward does.  dQ is summed over all key tiles
//   inside one workgroup, so it needs neither atomic adds nor a reduction
//   order (the determinism concern of FlashAttention-4 (papercache summary),
//   section 3.2.4).
//
// Both kernels write their gradients through LDS (each wave's rows there,
// then whole rows to HBM, 16 bytes per lane) rather than as the 8-byte
// pieces of 32 rows their accumulator layouts hold.
//
// Head dimensions 64 and 128 (template parameter D of every kernel).  LDS
// tiles hold rows of D bf16 in groups of 16 rows, each row starting
// at a staggered 16-byte unit of its group (the layout is described at
// row_slot below): 16-lane row reads and transpose reads meet no bank twice,
// and every read is one per-lane base address plus a compile-time offset,
// which keeps the kernels' address registers few.

#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstddef>
#include <cstdint>
#include <mutex>

#include "attn.h"
#include "cdna4.h"

namespace {

// Race check (as in the forward): a library built with -DATTN_FORCE_SAFE=1
// keeps every arithmetic step and its order, but the two wave groups of both
// ping-pong kernels run in lockstep instead of half a period apart, and every
// workgroup barrier waits first for all of the wave's outstanding memory
// operations.  Its gradients must equal the tuned build's bit for bit.
#ifndef ATTN_FORCE_SAFE
#define ATTN_FORCE_SAFE 0
#endif
constexpr bool kForceSafe = ATTN_FORCE_SAFE != 0;

// Head dimensions D of the backward kernels: 64 and 128.
constexpr int kBwThreads = 256;         // 4 waves
constexpr int kKeysPerWg = 128;         // dK/dV kernel: keys per workgroup
constexpr int kQStep = 32;              // dK/dV kernel: query rows per step

struct BwdParams {
  const __bf16* q;
  const __bf16* k;
  const __bf16* v;
  const __bf16* dout;
  const float* lse2;    // workspace: LSE * log2(e), +inf for empty rows, [B, Hq, Nq]
  const float* delta;   // workspace: <dO, O>, [B, Hq, Nq]
  __bf16* dq;
  __bf16* dk;
  __bf16* dv;
  const int32_t* seqlens_k;   // batched form: valid keys per batch element, may be null
  const int32_t* cu_q;        // packed form: sequence offsets into the rows, else null
  const int32_t* cu_k;
  const int32_t* seq_order;   // packed form: work order of the sequences, may be null
  int B, Hq, Hkv, G, Nq, Nk;  // packed form: B = sequences, Nq/Nk = the longest lengths
  long Tq;                    // packed form: total query rows (the LSE row stride per head)
  int nblk;             // key blocks (dK/dV) or query blocks (dQ) per (batch, head)
  int paired;           // 1: a workgroup runs the i-th and (n-1-i)-th item of a unit of n
  int pack;             // dQ: query heads of one KV group per workgroup (1, 2, 4 or 8)
  float c;              // scale * log2(e)
  float scale;
};

// Rows of one work unit (batch element, or sequence of a packed batch).
struct UnitRows {
  long q0, k0;    // first query / key row in the row-major arrays
  int nq, nk;     // valid queries and keys
  int k_write;    // keys whose dK, dV rows this unit writes
  long lse0;      // LSE / D index of (head 0, row 0); head h adds lse_h * h
  long lse_h;
};

__device__ __forceinline__ UnitRows unit_rows(const BwdParams& p, int b) {
  UnitRows r;
  if (p.cu_q != nullptr) {
    const int z = p.seq_order != nullptr ? min(max(p.seq_order[b], 0), p.B - 1) : b;
    r.q0 = min(max(p.cu_q[z], 0), (int)p.Tq);  // rows stay inside the total_q rows
    r.k0 = p.cu_k[z];
    r.nq = min(min(max(p.cu_q[z + 1] - p.cu_q[z], 0), p.Nq), (int)(p.Tq - r.q0));
    r.nk = min(max(p.cu_k[z + 1] - p.cu_k[z], 0), p.Nk);
    r.k_write = r.nk;
    r.lse0 = r.q0;
    r.lse_h = p.Tq;
  } else {
    r.q0 = (long)b * p.Nq;
    r.k0 = (long)b * p.Nk;
    r.nq = p.Nq;
    r.nk = p.seqlens_k != nullptr ? min(max(p.seqlens_k[b], 0), p.Nk) : p.Nk;
    r.k_write = p.Nk;  // padded keys get zero gradients
    r.lse0 = (long)b * p.Hq * p.Nq;
    r.lse_h = p.Nq;
  }
  // all uniform over the workgroup: keep them in scalar registers
  auto u64 = [](long x) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(x >> 32));
    return static_cast<long>((static_cast<uint64_t>(hi) << 32) | lo);
  };
  r.q0 = u64(r.q0);
  r.k0 = u64(r.k0);
  r.lse0 = u64(r.lse0);
  r.lse_h = u64(r.lse_h);
  r.nq = __builtin_amdgcn_readfirstlane(r.nq);
  r.nk = __builtin_amdgcn_readfirstlane(r.nk);
  r.k_write = __builtin_amdgcn_readfirstlane(r.k_write);
  return r;
}

// Work items of a launch: item id w belongs to XCD w % 8 (the hardware sends
// workgroup id w there), and XCD x takes the items of its units in order,
// longest first under the causal mask.  When p.paired is set, workgroup w
// runs two items of one unit of n: the i-th and the (n-1-i)-th, which cost
// about the same under the causal mask, with one launch and one pipeline
// fill less than two workgroups; the hardware still deals the pairs
// dynamically.  Otherwise workgroup w runs item w.
template <class F>
__device__ __forceinline__ void run_items(const BwdParams& p, int n, F&& run_item) {
  if (p.paired) {
    const int xcd = blockIdx.x % kXcds, m = blockIdx.x / kXcds;
    const int u = m / (n / 2), i = m % (n / 2);
    run_item((u * n + i) * kXcds + xcd);
    __syncthreads();  // the first item's LDS reads are done before the second's stores
    run_item((u * n + n - 1 - i) * kXcds + xcd);
  } else {
    run_item(static_cast<int>(blockIdx.x));
  }
}

// LDS tile layout.  Rows (D bf16, D/8 16-byte units) come in groups of 16; a
// group spans 16 (D/8 + 1) units and its row r starts at unit (D/8 + 1) a(r),
// with a(r) = 4 (r % 4) + r / 4.  D/8 + 1 (17 or 9) is odd, so a 16-lane row
// read (rows r0..r0+15, one chunk) meets 16 distinct 16-byte bank groups, and
// a transpose read (rows r0 + 4g + m, m = 0..3, 64 contiguous bytes each)
// starts at 4 (D/8 + 1) m + const, four disjoint 64-byte bank ranges: neither
// conflicts.  Rows are contiguous, so every read is one per-lane base address
// plus a compile-time offset.
template <int D>
struct Lds {
  static constexpr int kChunks = D / 8;                   // 16-byte chunks per row
  static constexpr int kStride = kChunks + 1;             // units per row slot
  static constexpr int kGroupElems = 16 * kStride * 8;    // elements per group of 16 rows
  static constexpr int kRowElems = kGroupElems / 16;      // tile size per row (multiples of 16 rows)

  // 16-byte unit at which row r (0..15) of a group starts.
  static __device__ __forceinline__ int row_slot(int r) { return kStride * (4 * (r & 3) + (r >> 2)); }

  // Element offset of (row, 16-byte chunk) in a tile.
  static __device__ __forceinline__ int tile_off(int row, int chunk) {
    return kGroupElems * (row >> 4) + 8 * (row_slot(row & 15) + chunk);
  }

  // Row-operand read: lane l takes row r0 + l%32, elements 16*ks + 8*(l/32) .. +7
  // (r0 a multiple of 16).
  static __device__ __forceinline__ bf16x8 read_rows(const __bf16* t, int r0, int ks, int lane) {
    const int lane_off = kGroupElems * ((lane >> 4) & 1) + 8 * (row_slot(lane & 15) + (lane >> 5));
    return *reinterpret_cast<const bf16x8*>(t + kGroupElems * (r0 >> 4) + lane_off + 16 * ks);
  }

  // Transposed operand: rows r0 + {4g..4g+3} then r0 + {8+4g..8+4g+3} (g = lane/32), as the
  // k-elements, for column d0 + lane%32 of the operand (r0 a multiple of 16, d0 of 32).
  static __device__ __forceinline__ bf16x8 read_cols(const __bf16* t, int r0, int d0, int lane) {
    const int g = lane >> 5, m = (lane & 15) >> 2, u = lane & 3;
    // first of this lane's 4 columns: d0 + 16 ((lane/16) % 2) + 4u
    const __bf16* base = t + kGroupElems * (r0 >> 4) + d0 + 16 * ((lane >> 4) & 1) + 4 * u;
    return read_tr_pair(base + 8 * row_slot(4 * g + m), base + 8 * row_slot(8 + 4 * g + m));
  }
};

// Buffer descriptor over [base, base + bytes), both uniform over the wave.
// readfirstlane keeps them in scalar registers: a descriptor the compiler
// leaves in vector registers turns every load through it into a loop.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t uniform_rsrc(const void* base, int bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32));
  return __builtin_amdgcn_make_buffer_rsrc(
      reinterpret_cast<void*>((static_cast<uint64_t>(hi) << 32) | lo), (short)0,
      __builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// Global rows [row0, row0 + rows) of a [.., stride] bf16 array -> padded LDS tile.
// Loads are 16 bytes per lane, row-contiguous; rows >= valid read as zero.
template <int ROWS, int D>
struct TileCopy {
  static constexpr int kChunks = D / 8;
  static constexpr int kPer = ROWS * kChunks / kBwThreads;  // chunks per thread
  static_assert(kPer * kBwThreads == ROWS * kChunks, "tile split");
  u32x4 r[kPer];
  __device__ __forceinline__ void load(const __bf16* base, long stride, int valid, int tid) {
    const __amdgpu_buffer_rsrc_t res = uniform_rsrc(base, max(valid, 0) * (int)(stride * 2));
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kBwThreads;
      const int row = c / kChunks, chunk = c % kChunks;
      r[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           res, (uint32_t)(row * stride * 2 + chunk * 16), 0, 0));
    }
  }
  __device__ __forceinline__ void store(__bf16* tile, int tid) const {
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
      const int c = tid + i * kBwThreads;
      *reinterpret_cast<u32x4*>(tile + Lds<D>::tile_off(c / kChunks, c % kChunks)) = r[i];
    }
  }
};

// ---------------------------------------------------------------------------
// D = <dO, O> and LSE in log2 units, one row per D/8 lanes.
// Packed form (B = 1, Nq = total rows): lse_rows points at the forward's LSE
// row count per head (cu_seqlens_q[num_seqs]); rows past it belong to no
// sequence and are skipped.  Batched form: lse_rows is null.
template <int D>
__global__ __launch_bounds__(256) void bwd_preprocess(const __bf16* o, const __bf16* dout,
                                                      const float* lse, float* lse2, float* delta,
                                                      int B, int Hq, int Nq,
                                                      const int32_t* lse_rows) {
  constexpr int kLanes = D / 8;            // lanes per row
  constexpr int kRows = 256 / kLanes;      // rows per block
  const long rows = (long)B * Nq * Hq;
  const long row = (long)blockIdx.x * kRows + (threadIdx.x / kLanes);  // row of [B, Nq, Hq]
  const int sub = threadIdx.x % kLanes;
  float acc = 0.f;
  if (row < rows) {
    const bf16x8 a = *reinterpret_cast<const bf16x8*>(o + row * D + sub * 8);
    const bf16x8 b = *reinterpret_cast<const bf16x8*>(dout + row * D + sub * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) acc += (float)a[e] * (float)b[e];
  }
#pragma unroll
  for (int off = kLanes / 2; off >= 1; off >>= 1) acc += __shfl_xor(acc, off, kLanes);
  if (row < rows && sub == 0) {
    const int h = (int)(row % Hq);
    const long bi = row / Hq;
    const int i = (int)(bi % Nq);
    const int b = (int)(bi / Nq);
    const long out = ((long)b * Hq + h) * Nq + i;
    long in = out;
    if (lse_rows != nullptr) {
      const int n = min(max(*lse_rows, 0), Nq);
      if (i >= n) return;
      in = (long)h * n + i;
    }
    const float l = lse[in];
    delta[out] = acc;
    lse2[out] = (l == -INFINITY) ? INFINITY : l * kLog2e;
  }
}

// ---------------------------------------------------------------------------
// dK, dV with two wave groups in ping-pong.  8 waves own 128 keys of one
// (batch, KV head); waves w and w+4 share a SIMD and the same 32 keys, and
// the two groups take alternate query steps (group g: steps g, g+2, ...).
// Each wave alternates an MFMA phase -- S and dP of its step i, then dV and
// dK of its step i-1 from the P and dS it packed in the previous phase --
// and a VALU phase (P and dS of step i, and the move of its group's next
// Q / dO tile into LDS); group 1 runs half a period behind group 0, so one
// wave of each SIMD feeds the matrix core while the other computes (the
// ping-pong of FlashAttention-4 (papercache summary), section 3.1.2, in
// CDNA form).  At the end the two groups' partial dK, dV are added through
// LDS in a fixed order.
constexpr int kBwPpThreads = 512;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwPpThreads, 1) void bwd_dkdv_pp_kernel(BwdParams p) {
  using L = Lds<D>;
  constexpr int kRowElems = L::kRowElems;
  constexpr int TD = D / 32;  // 32-wide d blocks of dK^T, dV^T
  __shared__ __attribute__((aligned(1024))) __bf16 kv_t[2 * kKeysPerWg * kRowElems];  // K, then V
  __shared__ __attribute__((aligned(1024))) __bf16 q_t[2][2][kQStep * kRowElems];  // [group][buffer]
  __shared__ __attribute__((aligned(1024))) __bf16 do_t[2][2][kQStep * kRowElems];
  __shared__ __attribute__((aligned(16))) float st_t[2][2][2 * kQStep];       // lse2, then D

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gtid = tid & (kBwThreads - 1);  // thread index within the group
  const int g = lane >> 5;
  const __bf16* k_t = kv_t;
  const __bf16* v_t = kv_t + kKeysPerWg * kRowElems;

  run_items(p, p.nblk, [&](const int id) __attribute__((always_inline)) {
    const int units = p.B * p.Hkv;
    const int x = id % kXcds, rr = id / kXcds;
    const int u = (rr / p.nblk) * kXcds + x;
    if (u >= units) return;  // grid padding; uniform over the workgroup
    const int kb = rr % p.nblk;
    const int b = u / p.Hkv, hkv = u % p.Hkv;
    const UnitRows ur = unit_rows(p, b);
    const int nk = ur.nk, nq = ur.nq;
    const int k0 = kb * kKeysPerWg;
    if (k0 >= ur.k_write) return;  // a packed sequence shorter than the longest; uniform
    const long kv_stride = (long)p.Hkv * D;
    const long q_stride = (long)p.Hq * D;

    // every tile buffer starts finite (periods without a step multiply zeros by
    // it); the barrier orders these stores before the first tile stores below
    for (int i = tid; i < 2 * 2 * kQStep * kRowElems / 8; i += kBwPpThreads) {
      reinterpret_cast<u32x4*>(&q_t[0][0][0])[i] = u32x4{};
      reinterpret_cast<u32x4*>(&do_t[0][0][0])[i] = u32x4{};
    }
    __syncthreads();
    {  // K (group 0) and V (group 1) of the block
      TileCopy<kKeysPerWg, D> c;
      const __bf16* src = (grp == 0 ? p.k : p.v) + (ur.k0 + k0) * kv_stride + (long)hkv * D;
      // an opaque copy of the thread index: the copy's lane addresses are
      // recomputed per work item instead of being kept across the loop
      int gt = gtid;
      asm volatile("" : "+v"(gt));
      c.load(src, kv_stride, min(nk - k0, kKeysPerWg), gt);
      c.store(kv_t + grp * kKeysPerWg * kRowElems, gt);
    }

    const int wk0 = k0 + (wave & 3) * 32;  // this wave's first key
    const int key = wk0 + (lane & 31);
    f32x16 dk_acc[TD], dv_acc[TD];
#pragma unroll
    for (int t = 0; t < TD; ++t) dk_acc[t] = dv_acc[t] = f32x16{};

    const int s0 = CAUSAL ? (k0 / kQStep) : 0;
    const int nsteps_h = (nq + kQStep - 1) / kQStep - s0;
    const int nsteps = nk > k0 ? max(nsteps_h, 0) * p.G : 0;
    const int n_mine = (nsteps - grp + 1) / 2;   // this group's steps: grp, grp+2, ...
    const int n_per = (nsteps + 1) / 2 + 1;      // periods, the same for both groups

    TileCopy<kQStep, D> qc, dc;
    float stat = 0.f;
    // first query row and head of this group's i-th step.  Steps run from the
    // last query rows back to the first, the G heads of a row block innermost:
    // the workgroups of one (batch, KV head), which run side by side on one XCD,
    // then read the same Q and dO rows at about the same time, from L2.
    auto step_rows = [&](int i) {
      const int s = 2 * i + grp;
      return make_int2((s0 + nsteps_h - 1 - s / p.G) * kQStep, hkv * p.G + s % p.G);
    };
    auto fetch = [&](int i) {
      const int2 r = step_rows(i);
      const long rowbase = (ur.q0 + r.x) * q_stride + (long)r.y * D;
      const int valid = min(nq - r.x, kQStep);
      qc.load(p.q + rowbase, q_stride, valid, gtid);
      dc.load(p.dout + rowbase, q_stride, valid, gtid);
      if (gtid < 2 * kQStep) {
        const int row = r.x + (gtid & 31);
        const long sidx = ur.lse0 + ur.lse_h * r.y + row;
        stat = (row < nq) ? (gtid < kQStep ? p.lse2[sidx] : p.delta[sidx])
                            : (gtid < kQStep ? INFINITY : 0.f);
      }
    };
    auto put = [&](int buf) {
      qc.store(q_t[grp][buf], gtid);
      dc.store(do_t[grp][buf], gtid);
      if (gtid < 2 * kQStep) st_t[grp][buf][gtid] = stat;
    };
    auto barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kForceSafe) __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 s_acc = {}, dp_acc = {};
    u32x4 p_pk[2] = {}, ds_pk[2] = {};
    // MFMA phase slices, in groups of four for i = 0 .. D/16 - 1: S (k-slice
    // i), dV, dP (k-slice i), dK, the last two for 16 queries qs = i / TD and
    // 32 dimensions t = i % TD.  S and dP read two row operands each, dV and dK
    // one transposed operand, so the LDS demand stays even over the phase.
    // Each slice's operands are read kAhead slices before its MFMA; scheduling
    // barriers between the slices keep that order.
    constexpr int kSlices = 4 * (D / 16), kAhead = 3;
    struct Opnd {
      bf16x8 a, b;
    };
    // One period: MFMA phase, barrier, VALU phase, barrier.
    auto period = [&](int i, auto par) {
      constexpr int B0 = decltype(par)::value;  // i % 2: buffer of step i
      const __bf16* qt = q_t[grp][B0];
      const __bf16* dt = do_t[grp][B0];
      const __bf16* qo = q_t[grp][B0 ^ 1];  // step i-1
      const __bf16* dto = do_t[grp][B0 ^ 1];
      const int kr0 = (wave & 3) * 32;
      auto operand = [&](auto I) __attribute__((always_inline)) -> Opnd {
        constexpr int sl = decltype(I)::value, n = sl >> 2, kind = sl & 3;
        if constexpr (kind == 0) return {L::read_rows(qt, 0, n, lane), L::read_rows(k_t, kr0, n, lane)};
        else if constexpr (kind == 2) return {L::read_rows(dt, 0, n, lane), L::read_rows(v_t, kr0, n, lane)};
        else if constexpr (kind == 1) return {L::read_cols(dto, 16 * (n / TD), 32 * (n % TD), lane), bf16x8{}};
        else return {L::read_cols(qo, 16 * (n / TD), 32 * (n % TD), lane), bf16x8{}};
      };
      // ---- MFMA phase
      Opnd opnd[kAhead];
      static_for<0, kAhead>([&](auto I) __attribute__((always_inline)) {
        opnd[decltype(I)::value] = operand(I);
      });
      static_for<0, kSlices>([&](auto I) __attribute__((always_inline)) {
        constexpr int sl = decltype(I)::value, n = sl >> 2, kind = sl & 3;
        const Opnd o = opnd[sl % kAhead];
        if constexpr (sl + kAhead < kSlices) opnd[sl % kAhead] = operand(std::integral_constant<int, sl + kAhead>{});
        if constexpr (kind == 0)
          s_acc = mfma32(o.a, o.b, n == 0 ? f32x16{} : s_acc);
        else if constexpr (kind == 2)
          dp_acc = mfma32(o.a, o.b, n == 0 ? f32x16{} : dp_acc);
        else if constexpr (kind == 1)
          dv_acc[n % TD] = mfma32(o.a, __builtin_bit_cast(bf16x8, p_pk[n / TD]), dv_acc[n % TD]);
        else
          dk_acc[n % TD] = mfma32(o.a, __builtin_bit_cast(bf16x8, ds_pk[n / TD]), dk_acc[n % TD]);
        __builtin_amdgcn_sched_barrier(0);
      });
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      // ---- VALU phase: P, dS of step i (zero when this group has no step i);
      // this group's step i+1 is loaded meanwhile and stored into the buffer
      // step i-1 used (its last reader was the MFMA phase just finished).  A
      // step whose rows all see all of this wave's keys skips the mask.
      const bool more = i + 1 < n_mine;
      if (more) fetch(i + 1);
      if (i < n_mine) {
        const int i0 = step_rows(i).x;
        const float* l2t = st_t[grp][B0];
        const float* ddt = st_t[grp][B0] + kQStep;
        const bool full = wk0 + 32 <= nk && (!CAUSAL || wk0 + 31 <= i0);
        // Row 8 r4 + 4 g + e of the step sees this lane's key when 8 r4 + e
        // >= u (one compare per score): the key lies below nk and, causal,
        // not past the row.
        const int u = key < nk ? (CAUSAL ? key - i0 - 4 * g : INT_MIN) : INT_MAX;
        auto block = [&](bool masked) __attribute__((always_inline)) {
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const int qi = 8 * r4 + 4 * g;
            const float4 l2 = *reinterpret_cast<const float4*>(l2t + qi);
            const float4 dd = *reinterpret_cast<const float4*>(ddt + qi);
            float pv[4], dsv[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * r4 + e;
              const float lv = e == 0 ? l2.x : e == 1 ? l2.y : e == 2 ? l2.z : l2.w;
              const float dv_ = e == 0 ? dd.x : e == 1 ? dd.y : e == 2 ? dd.z : dd.w;
              const bool vis = !masked || 8 * r4 + e >= u;
              const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(s_acc[r], p.c, -lv)) : 0.f;
              pv[e] = pe;
              dsv[e] = pe * (dp_acc[r] - dv_);
            }
            const bf16x2 p01 = {(__bf16)pv[0], (__bf16)pv[1]}, p23 = {(__bf16)pv[2], (__bf16)pv[3]};
            const bf16x2 d01 = {(__bf16)dsv[0], (__bf16)dsv[1]}, d23 = {(__bf16)dsv[2], (__bf16)dsv[3]};
            p_pk[r4 >> 1][2 * (r4 & 1)] = __builtin_bit_cast(uint32_t, p01);
            p_pk[r4 >> 1][2 * (r4 & 1) + 1] = __builtin_bit_cast(uint32_t, p23);
            ds_pk[r4 >> 1][2 * (r4 & 1)] = __builtin_bit_cast(uint32_t, d01);
            ds_pk[r4 >> 1][2 * (r4 & 1) + 1] = __builtin_bit_cast(uint32_t, d23);
          }
        };
        if (full)
          block(false);
        else
          block(true);
      } else {
        p_pk[0] = p_pk[1] = ds_pk[0] = ds_pk[1] = u32x4{};
      }
      if (more) put(B0 ^ 1);
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
    };

    if (n_mine > 0) {
      fetch(0);
      put(0);
    }
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __syncthreads();
    if (!kForceSafe && grp == 1) barrier();  // group 1 runs half a period behind
    int i = 0;
    for (; i + 1 < n_per; i += 2) {
      period(i, std::integral_constant<int, 0>{});
      period(i + 1, std::integral_constant<int, 1>{});
    }
    if (i < n_per) period(i, std::integral_constant<int, 0>{});
    if (!kForceSafe && grp == 0) barrier();
    __syncthreads();

    // ---- combine: group 1's partial sums go through LDS (fp32, [key][d]) into group 0's
    // [key][d] fp32 with rows padded by 16 bytes, so 16 lanes on 16 keys meet distinct banks
    constexpr int kRedPitch = D + 4;
    static_assert(sizeof(kv_t) >= kKeysPerWg * kRedPitch * sizeof(float), "reduction buffer");
    float* red = reinterpret_cast<float*>(kv_t);  // K and V are no longer needed
    // Lane quantities of the reduction and the stores, derived afresh from an
    // opaque copy of the thread index so that the compiler does not keep them
    // live across the period loop.
    int tid_late = static_cast<int>(threadIdx.x);
    asm volatile("" : "+v"(tid_late));
    const int lane_l = tid_late & 63, g_l = lane_l >> 5;
    const int kl = (wave & 3) * 32 + (lane_l & 31);   // key within the block
    auto xfer = [&](f32x16* acc, bool add) {
#pragma unroll
      for (int t = 0; t < TD; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          float4* slot = reinterpret_cast<float4*>(red + kl * kRedPitch + 32 * t + 8 * r4 + 4 * g_l);
          if (add) {
            const float4 o = *slot;
            acc[t][4 * r4 + 0] += o.x;
            acc[t][4 * r4 + 1] += o.y;
            acc[t][4 * r4 + 2] += o.z;
            acc[t][4 * r4 + 3] += o.w;
          } else {
            *slot = make_float4(acc[t][4 * r4 + 0], acc[t][4 * r4 + 1], acc[t][4 * r4 + 2],
                                acc[t][4 * r4 + 3]);
          }
        }
    };
    if (grp == 1) xfer(dk_acc, false);
    __syncthreads();
    if (grp == 0) xfer(dk_acc, true);
    __syncthreads();
    if (grp == 1) xfer(dv_acc, false);
    __syncthreads();
    if (grp == 0) xfer(dv_acc, true);

    // dK and dV leave through LDS (the Q and dO tiles are no longer read): a
    // lane's accumulators hold 4-column pieces of one key row, so storing
    // them directly scatters every store instruction over 32 rows.  Each wave
    // of group 0 writes its 32 keys' rows, in bf16, row-major (16-byte chunk c
    // of row r at chunk c XOR (r % (D/8))) into its part of the Q tiles (dK)
    // and the dO tiles (dV), then stores whole rows with 16-byte stores.
    if (grp == 0) {
      constexpr int kOChunks = D / 8;
      static_assert(64 % kOChunks == 0 && 32 % (64 / kOChunks) == 0, "row passes");
      static_assert(sizeof(q_t) >= 4 * 32 * D * sizeof(__bf16) &&
                        sizeof(do_t) >= 4 * 32 * D * sizeof(__bf16),
                    "dK, dV staging");
      const int l32 = lane_l & 31;
      __bf16* const sk = &q_t[0][0][0] + (wave & 3) * (32 * D);
      __bf16* const sd = &do_t[0][0][0] + (wave & 3) * (32 * D);
#pragma unroll
      for (int t = 0; t < TD; ++t)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          bf16x4 a, c;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a[e] = (__bf16)(dk_acc[t][4 * r4 + e] * p.scale);
            c[e] = (__bf16)dv_acc[t][4 * r4 + e];
          }
          const int off = l32 * D + (((t * 4 + r4) ^ (l32 % kOChunks)) * 8) + 4 * g_l;
          *reinterpret_cast<bf16x4*>(sk + off) = a;
          *reinterpret_cast<bf16x4*>(sd + off) = c;
        }
      // the wave's LDS writes precede its reads of other lanes' data
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int wkey0 = k0 + (wave & 3) * 32;  // this wave's first key
      const long row0 = (ur.k0 + wkey0) * kv_stride + (long)hkv * D;
      constexpr int kRowsPerPass = 64 / kOChunks;
      const int cc = lane_l % kOChunks;
#pragma unroll
      for (int i = 0; i < 32 / kRowsPerPass; ++i) {
        const int r = i * kRowsPerPass + lane_l / kOChunks;
        const int off = r * D + (cc ^ (r % kOChunks)) * 8;
        const u32x4 a = *reinterpret_cast<const u32x4*>(sk + off);
        const u32x4 c = *reinterpret_cast<const u32x4*>(sd + off);
        if (wkey0 + r < ur.k_write && wkey0 + r < k0 + kKeysPerWg) {
          *reinterpret_cast<u32x4*>(p.dk + row0 + r * kv_stride + cc * 8) = a;
          *reinterpret_cast<u32x4*>(p.dv + row0 + r * kv_stride + cc * 8) = c;
        }
      }
    }
  });
}

// ---------------------------------------------------------------------------
// dQ with two wave groups in ping-pong: 8 waves own 256 query rows of one
// head (wave w: rows 32 * (2(w%4) + w/4) .. +31, so the two waves of a SIMD
// hold adjacent rows); K and V stream in tiles of 32 keys.  Each wave
// alternates an MFMA phase -- S and dP of tile j, then dQ^T += K^T dS^T of
// tile j-1 -- and a VALU phase (P, dS of tile j); group 1 runs half a period
// behind.  Group 0 moves V tiles (two buffers: V_j is read only in phase j),
// group 1 moves K tiles (four buffers: K_j is read again for dQ one period
// later); each stores the next tile and loads the one after while its MFMAs
// run.
constexpr int kDqTile = 32;
constexpr int kDqRows = 256;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwPpThreads, 1) void bwd_dq_pp_kernel(BwdParams p) {
  using L = Lds<D>;
  constexpr int kRowElems = L::kRowElems;
  constexpr int TD = D / 32;  // 32-wide d blocks of dQ^T
  constexpr int KS = D / 16;  // 16-deep d slices of S^T and dP^T
  __shared__ __attribute__((aligned(1024))) __bf16 k_t[4][kDqTile * kRowElems];
  __shared__ __attribute__((aligned(1024))) __bf16 v_t[2][kDqTile * kRowElems];
  // Each wave's dQ rows on their way to HBM (see the end of an item).
  constexpr int kWaves = kBwPpThreads / 64;
  __shared__ __attribute__((aligned(1024))) __bf16 dq_lds[kWaves * 32 * D];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;
  const int gtid = tid & (kBwThreads - 1);
  const int g = lane >> 5;

  run_items(p, p.nblk * (p.G / p.pack), [&](const int id) __attribute__((always_inline)) {
    const int units = p.B * p.Hkv;
    // The workgroup takes P = p.pack query heads of the KV group, 256 / P rows
    // of each: row chunk c = 2 (w % 4) + w / 4 of wave w holds rows
    // (c % cph) * 32 .. +31 of head gi + c / cph, so the two waves of a SIMD
    // share their causal extent, and under the causal mask the workgroup's
    // rows cross fewer key tiles on the diagonal (as in the forward).
    const int per_unit = p.nblk * (p.G / p.pack);
    const int x = id % kXcds, rr = id / kXcds;
    const int u = (rr / per_unit) * kXcds + x;
    if (u >= units) return;
    const int item = rr % per_unit;
    const int groups = p.G / p.pack;
    const int qbi = item / groups, gi = (item % groups) * p.pack;
    const int qb = CAUSAL ? (p.nblk - 1 - qbi) : qbi;
    const int b = u / p.Hkv, hkv = u % p.Hkv;
    const int chunk = 2 * (wave & 3) + grp;
    const int cph = 8 / p.pack;                 // 32-row chunks per head
    const int rows_h = 32 * cph;                // query rows per head
    const int h = hkv * p.G + gi + chunk / cph;
    const UnitRows ur = unit_rows(p, b);
    const int nk = ur.nk, nq = ur.nq;

    const long kv_stride = (long)p.Hkv * D;
    const long q_stride = (long)p.Hq * D;
    const int q0 = qb * rows_h;
    if (q0 >= nq) return;  // a packed sequence shorter than the longest; uniform
    const int wrow0 = q0 + 32 * (chunk % cph);
    const int qrow = wrow0 + (lane & 31);
    bf16x8 qf[KS], df[KS];
    const long qoff = (ur.q0 + qrow) * q_stride + (long)h * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      qf[ks] = qrow < nq ? *reinterpret_cast<const bf16x8*>(p.q + qoff + 16 * ks + 8 * g) : bf16x8{};
      df[ks] = qrow < nq ? *reinterpret_cast<const bf16x8*>(p.dout + qoff + 16 * ks + 8 * g) : bf16x8{};
    }
    const long sidx = ur.lse0 + ur.lse_h * h + qrow;
    const float l2 = qrow < nq ? p.lse2[sidx] : INFINITY;
    const float dd = qrow < nq ? p.delta[sidx] : 0.f;
    __builtin_amdgcn_s_waitcnt(kWaitVm0);  // operands ready before any tile load is in flight

    int kv_end = nk;
    if (CAUSAL) kv_end = min(nk, q0 + rows_h);
    const int n_tiles = (kv_end + kDqTile - 1) / kDqTile;
    const __bf16* src = (grp == 0 ? p.v : p.k) + ur.k0 * kv_stride + (long)hkv * D;

    // every buffer starts finite (the first dQ step multiplies zeros by K)
    for (int i = tid; i < 4 * kDqTile * kRowElems / 8; i += kBwPpThreads)
      reinterpret_cast<u32x4*>(&k_t[0][0])[i] = u32x4{};
    for (int i = tid; i < 2 * kDqTile * kRowElems / 8; i += kBwPpThreads)
      reinterpret_cast<u32x4*>(&v_t[0][0])[i] = u32x4{};
    __syncthreads();

    TileCopy<kDqTile, D> stage;
    auto fetch = [&](int j) {
      const int j0 = j * kDqTile;
      stage.load(src + (long)j0 * kv_stride, kv_stride, min(kv_end - j0, kDqTile), gtid);
    };
    auto kbuf = [&](auto I) -> __bf16* { return k_t[decltype(I)::value & 3]; };
    auto vbuf = [&](auto I) -> __bf16* { return v_t[decltype(I)::value & 1]; };
    auto barrier = [&]() {
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (kForceSafe) __builtin_amdgcn_s_waitcnt(0);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
    };

    f32x16 acc[TD];
#pragma unroll
    for (int t = 0; t < TD; ++t) acc[t] = f32x16{};
    f32x16 s_acc = {}, dp_acc = {};
    u32x4 ds_pk[2] = {};

    // MFMA phase slices: 0 .. 2 KS - 1 are S and dP of tile j, alternating (one
    // K or V row operand each), then 2 TD slices of dQ of tile j-1 (one K^T
    // operand each).  Each slice's LDS operand is read kAhead slices before its
    // MFMA; scheduling barriers between the slices keep that order.  The tile
    // move sits after slice kMoveAt, half-way.
    constexpr int kSD = 2 * KS;
    constexpr int kSlices = kSD + 2 * TD, kAhead = 4, kMoveAt = kSlices / 2;
    auto period = [&](int j, auto J) {
      constexpr int j4 = decltype(J)::value;  // j % 4
      const __bf16* kt = kbuf(std::integral_constant<int, j4>{});
      const __bf16* vt = vbuf(std::integral_constant<int, j4>{});
      const __bf16* kto = kbuf(std::integral_constant<int, j4 + 3>{});  // tile j-1
      auto operand = [&](auto I) __attribute__((always_inline)) -> bf16x8 {
        constexpr int i = decltype(I)::value;
        if constexpr (i < kSD) return L::read_rows((i & 1) ? vt : kt, 0, i >> 1, lane);
        else return L::read_cols(kto, 16 * ((i - kSD) / TD), 32 * ((i - kSD) % TD), lane);
      };
      // ---- MFMA phase, with this group's tile move after slice kMoveAt
      bf16x8 opnd[kAhead];
      static_for<0, kAhead>([&](auto I) __attribute__((always_inline)) {
        opnd[decltype(I)::value] = operand(I);
      });
      static_for<0, kSlices>([&](auto I) __attribute__((always_inline)) {
        constexpr int i = decltype(I)::value;
        const bf16x8 a = opnd[i % kAhead];
        if constexpr (i + kAhead < kSlices) opnd[i % kAhead] = operand(std::integral_constant<int, i + kAhead>{});
        if constexpr (i < kSD) {
          constexpr int ks = i >> 1;
          if constexpr (i & 1)
            dp_acc = mfma32(a, df[ks], ks == 0 ? f32x16{} : dp_acc);
          else
            s_acc = mfma32(a, qf[ks], ks == 0 ? f32x16{} : s_acc);
        } else {
          constexpr int hh = (i - kSD) / TD, t = (i - kSD) % TD;
          acc[t] = mfma32(a, __builtin_bit_cast(bf16x8, ds_pk[hh]), acc[t]);
        }
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (i == kMoveAt) {
          // group 0 stores V_{j+1} over V_{j-1}, group 1 K_{j+1} over K_{j-3}
          if (j + 1 < n_tiles) {
            stage.store(grp == 0 ? vbuf(std::integral_constant<int, j4 + 1>{})
                                 : kbuf(std::integral_constant<int, j4 + 1>{}),
                        gtid);
            if (j + 2 < n_tiles) fetch(j + 2);
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      });
      __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
      barrier();
      // ---- VALU phase: P, dS of tile j (zero past the last tile).  A tile whose
      // keys all are visible to all of this wave's rows skips the mask.
      if (j < n_tiles) {
        const int j0 = j * kDqTile;
        const bool full = j0 + kDqTile <= nk && (!CAUSAL || j0 + kDqTile - 1 <= wrow0);
        // keys below key_lim are visible to this lane's row; score r of the
        // lane is key j0 + 4 g + (a compile-time offset): one compare per score
        const int t = (CAUSAL ? min(nk, qrow + 1) : nk) - j0 - 4 * g;
        auto dsval = [&](int r, bool masked) __attribute__((always_inline)) {
          const bool vis = !masked || 8 * (r >> 2) + (r & 3) < t;
          const float pe = vis ? __builtin_amdgcn_exp2f(fmaf(s_acc[r], p.c, -l2)) : 0.f;
          return pe * (dp_acc[r] - dd);
        };
        if (full) {
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const bf16x2 pk = {(__bf16)dsval(r, false), (__bf16)dsval(r + 1, false)};
            ds_pk[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
          }
        } else {
#pragma unroll
          for (int r = 0; r < 16; r += 2) {
            const bf16x2 pk = {(__bf16)dsval(r, true), (__bf16)dsval(r + 1, true)};
            ds_pk[r >> 3][(r & 7) >> 1] = __builtin_bit_cast(uint32_t, pk);
          }
        }
      } else {
        ds_pk[0] = ds_pk[1] = u32x4{};
      }
      barrier();
    };

    if (n_tiles > 0) {
      fetch(0);
      stage.store(grp == 0 ? v_t[0] : k_t[0], gtid);
    }
    if (n_tiles > 1) fetch(1);
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __syncthreads();
    if (!kForceSafe && grp == 1) barrier();  // group 1 runs half a period behind
    int j = 0;
    for (; j + 3 <= n_tiles; j += 4) {
      period(j, std::integral_constant<int, 0>{});
      period(j + 1, std::integral_constant<int, 1>{});
      period(j + 2, std::integral_constant<int, 2>{});
      period(j + 3, std::integral_constant<int, 3>{});
    }
    if (j <= n_tiles) period(j, std::integral_constant<int, 0>{});
    if (j + 1 <= n_tiles) period(j + 1, std::integral_constant<int, 1>{});
    if (j + 2 <= n_tiles) period(j + 2, std::integral_constant<int, 2>{});
    if (!kForceSafe && grp == 0) barrier();

    // dQ leaves through LDS: a lane's accumulator holds 4-column pieces of one
    // row, so storing it directly scatters every store instruction over 32
    // rows.  Each wave writes its 32 x D block, scaled, in bf16, row-major into
    // its own part of dq_lds (16-byte chunk c of row r at chunk c XOR (r %
    // (D/8)), conflict-free for the column writes and the row reads), then
    // stores whole rows with 16-byte stores.
    constexpr int kOChunks = D / 8;
    static_assert(64 % kOChunks == 0 && 32 % (64 / kOChunks) == 0, "dQ row passes");
    const int l32 = lane & 31;
    __bf16* const ost = dq_lds + wave * (32 * D);
#pragma unroll
    for (int t = 0; t < TD; ++t)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        bf16x4 a;
#pragma unroll
        for (int e = 0; e < 4; ++e) a[e] = (__bf16)(acc[t][4 * r4 + e] * p.scale);
        const int chk = (t * 4 + r4) ^ (l32 % kOChunks);  // columns 32 t + 8 r4 .. +7
        *reinterpret_cast<bf16x4*>(ost + l32 * D + chk * 8 + 4 * g) = a;
      }
    // the wave's LDS writes precede its reads of other lanes' data
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __bf16* const dq0 = p.dq + (ur.q0 + wrow0) * q_stride + (long)h * D;
    constexpr int kRowsPerPass = 64 / kOChunks;
    const int cc = lane % kOChunks;
#pragma unroll
    for (int i = 0; i < 32 / kRowsPerPass; ++i) {
      const int r = i * kRowsPerPass + lane / kOChunks;
      const u32x4 v = *reinterpret_cast<const u32x4*>(ost + r * D + (cc ^ (r % kOChunks)) * 8);
      if (wrow0 + r < nq) *reinterpret_cast<u32x4*>(dq0 + r * q_stride + cc * 8) = v;
    }
  });
}

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) % 16) == 0; }

int launched() {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  return ATTN_OK;
}

// Launches preprocess, dK/dV and dQ for the units p describes.  The LSE and
// D workspace rows are [pre_b, Hq, pre_nq] (batched: B, Nq; packed: 1, Tq).
template <int D>
int launch_backward_d(BwdParams p, const __bf16* o, const float* lse, int pre_b, long pre_nq,
                      const int32_t* lse_rows, bool need_q, bool need_k, bool causal,
                      hipStream_t st) {
  constexpr long kPreRows = 256 / (D / 8);  // rows per preprocess block
  const long units8 = ((long)p.B * p.Hkv + kXcds - 1) / kXcds * kXcds;
  const int nblk_k = (p.Nk + kKeysPerWg - 1) / kKeysPerWg;
  // dQ workgroups take the largest power of two up to 8 dividing G of a KV
  // group's query heads together (256 / pack rows of each).
  p.pack = p.G % 8 == 0 ? 8 : p.G % 4 == 0 ? 4 : p.G % 2 == 0 ? 2 : 1;
  const int rows_q = kDqRows / p.pack;
  const int nblk_q = (p.Nq + rows_q - 1) / rows_q;
  const long grid_k = units8 * nblk_k, grid_q = units8 * nblk_q * (p.G / p.pack);
  const long rows = (long)pre_b * pre_nq * p.Hq;
  const long grid_pre = (rows + kPreRows - 1) / kPreRows;
  if (grid_k > INT_MAX || grid_q > INT_MAX || grid_pre > INT_MAX) return ATTN_ERR_TOO_LARGE;
  float* lse2 = const_cast<float*>(p.lse2);
  float* delta = const_cast<float*>(p.delta);
  // Paired items (run_items) for the batched form with at most 8192 keys,
  // as in the forward: the packed form's differing lengths make pairs uneven
  // (measured 1 % slower), and longer sequences gained nothing.
  const bool packed = p.cu_q != nullptr || p.Nk > 8192;
  if (need_q) {
    hipLaunchKernelGGL(bwd_preprocess<D>, dim3((unsigned)grid_pre), dim3(256), 0, st, o, p.dout,
                       lse, lse2, delta, pre_b, p.Hq, (int)pre_nq, lse_rows);
    if (int rc = launched()) return rc;
  }
  if (need_k) {
    p.nblk = nblk_k;
    p.paired = packed ? 0 : nblk_k % 2 == 0;
    const unsigned wgs = (unsigned)(p.paired ? grid_k / 2 : grid_k);
    if (causal)
      hipLaunchKernelGGL((bwd_dkdv_pp_kernel<D, true>), dim3(wgs), dim3(kBwPpThreads), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dkdv_pp_kernel<D, false>), dim3(wgs), dim3(kBwPpThreads), 0, st, p);
    if (int rc = launched()) return rc;
  }
  if (need_q) {
    p.nblk = nblk_q;
    p.paired = packed ? 0 : (nblk_q * (p.G / p.pack)) % 2 == 0;
    const unsigned wgs = (unsigned)(p.paired ? grid_q / 2 : grid_q);
    if (causal)
      hipLaunchKernelGGL((bwd_dq_pp_kernel<D, true>), dim3(wgs), dim3(kBwPpThreads), 0, st, p);
    else
      hipLaunchKernelGGL((bwd_dq_pp_kernel<D, false>), dim3(wgs), dim3(kBwPpThreads), 0, st, p);
    if (int rc = launched()) return rc;
  }
  return ATTN_OK;
}

int launch_backward(int d, const BwdParams& p, const __bf16* o, const float* lse, int pre_b,
                    long pre_nq, const int32_t* lse_rows, bool need_q, bool need_k, bool causal,
                    hipStream_t st) {
  if (d == 64)
    return launch_backward_d<64>(p, o, lse, pre_b, pre_nq, lse_rows, need_q, need_k, causal, st);
  return launch_backward_d<128>(p, o, lse, pre_b, pre_nq, lse_rows, need_q, need_k, causal, st);
}

}  // namespace

extern "C" size_t attn_bwd_workspace_size(int B, int Hq, int Nq) {
  if (B <= 0 || Hq <= 0 || Nq <= 0) return 0;
  return (size_t)2 * sizeof(float) * (size_t)B * (size_t)Hq * (size_t)Nq;
}

namespace {

// Host-side checks of the batched backward, except its workspace pointer.
// Sets *noop when there is nothing to compute.
int check_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv, int Nq,
              int Nk, int d, float scale, bool* noop) {
  *noop = false;
  if (B < 0 || Nq < 0 || Nk < 0) return ATTN_ERR_SIZE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_SIZE;  // any finite scale: P = exp2(s c - lse2)
  if (B == 0 || (Nq == 0 && Nk == 0)) {
    *noop = true;
    return ATTN_OK;
  }
  const bool need_q = Nq > 0, need_k = Nk > 0;
  if ((need_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) ||
      (need_q && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
                  dq == nullptr)))
    return ATTN_ERR_NULL;
  if ((need_q && (!aligned16(q) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
                  (reinterpret_cast<uintptr_t>(lse) % 4) != 0)) ||
      (need_k && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))))
    return ATTN_ERR_ALIGN;
  const long rows = (long)B * Nq * Hq;
  // Row counts stay within int; element offsets are 64-bit throughout.
  if (rows > INT_MAX || (long)B * Nk * Hkv > INT_MAX) return ATTN_ERR_TOO_LARGE;
  return ATTN_OK;
}

// Launches the batched backward with the LSE * log2(e) and D rows at `ws`
// (2 * B * Hq * Nq floats, every one written by the preprocess kernel before
// it is read).
int run_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* ws, int B, int Hq, int Hkv,
            int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
            void* stream) {
  const long rows = (long)B * Nq * Hq;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  BwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.dout = static_cast<const __bf16*>(dout);
  p.lse2 = ws;
  p.delta = ws + rows;
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.seqlens_k = seqlens_k;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = Nq;
  p.Nk = Nk;
  p.scale = scale;
  p.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return launch_backward(d, p, static_cast<const __bf16*>(o), lse, B, Nq, nullptr, Nq > 0, Nk > 0,
                         causal != 0, st);
}

// ---------------------------------------------------------------------------
// Allocation-free backward: the LSE * log2(e) and D rows live in a static
// device array instead of a caller workspace.  Each device holds its own copy
// of the array; host code reaches it only through the address
// hipGetSymbolAddress returns with that device current (the array's name is a
// host-side stand-in, not a device address), kept per device.  Calls on one
// device share the array, so calls that overlap on a device race; every
// entry a call reads is written by that call's preprocess kernel first, so
// nothing needs clearing between calls.
constexpr size_t kScratchBytes = size_t(32) << 20;                   // 32 MiB per device
constexpr long kScratchRows = long(kScratchBytes / (2 * sizeof(float)));  // (batch, head, row) triples
constexpr int kMaxDevices = 64;

static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Device address of this device's scratch (looked up once per device).
int scratch_of_current_device(float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    attn_detail::last_hip_error = static_cast<int>(e);
    return ATTN_ERR_LAUNCH;
  }
  if (dev < 0 || dev >= kMaxDevices) return ATTN_ERR_TOO_LARGE;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (scratch_ptr[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      attn_detail::last_hip_error = static_cast<int>(e);
      return ATTN_ERR_LAUNCH;
    }
    scratch_ptr[dev] = ptr;
  }
  *out = static_cast<float*>(scratch_ptr[dev]);
  return ATTN_OK;
}

}  // namespace

extern "C" int attn_bwd(const void* q, const void* k, const void* v, const void* o,
                        const float* lse, const void* dout, void* dq, void* dk, void* dv,
                        void* workspace, int B, int Hq, int Hkv, int Nq, int Nk, int d,
                        float scale, int causal, const int32_t* seqlens_k, void* stream) {
  bool noop = false;
  const int rc = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, &noop);
  if (rc != ATTN_OK || noop) return rc;
  if (Nq > 0 && workspace == nullptr) return ATTN_ERR_NULL;
  if (Nq > 0 && !aligned16(workspace)) return ATTN_ERR_ALIGN;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, static_cast<float*>(workspace), B, Hq, Hkv, Nq,
                 Nk, d, scale, causal, seqlens_k, stream);
}

extern "C" int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o,
                                const float* lse, const void* dout, void* dq, void* dk, void* dv,
                                int B, int Hq, int Hkv, int Nq, int Nk, int d, float scale,
                                int causal, const int32_t* seqlens_k, void* stream) {
  bool noop = false;
  const int rc = check_bwd(q, k, v, o, lse, dout, dq, dk, dv, B, Hq, Hkv, Nq, Nk, d, scale, &noop);
  if (rc != ATTN_OK || noop) return rc;
  if ((long)B * Hq * Nq > kScratchRows) return ATTN_ERR_SCRATCH;
  float* ws = nullptr;
  const int src = scratch_of_current_device(&ws);
  if (src != ATTN_OK) return src;
  return run_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, B, Hq, Hkv, Nq, Nk, d, scale, causal,
                 seqlens_k, stream);
}


extern "C" int attn_bwd_varlen_ordered(const void* q, const void* k, const void* v,
                                       const void* o, const float* lse, const void* dout, void* dq,
                                       void* dk, void* dv, void* workspace,
                                       const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                       int num_seqs, int total_q, int Hq, int Hkv,
                                       int max_seqlen_q, int max_seqlen_k, int d, float scale,
                                       int causal, const int32_t* seq_order, void* stream) {
  if (num_seqs < 0 || total_q < 0 || max_seqlen_q < 0 || max_seqlen_k < 0) return ATTN_ERR_SIZE;
  if (Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return ATTN_ERR_HEADS;
  if (d != 64 && d != 128) return ATTN_ERR_HEAD_DIM;
  if (!std::isfinite(scale)) return ATTN_ERR_SIZE;  // any finite scale: P = exp2(s c - lse2)
  if (num_seqs == 0 || (max_seqlen_q == 0 && max_seqlen_k == 0)) return ATTN_OK;
  if (cu_seqlens_q == nullptr || cu_seqlens_k == nullptr) return ATTN_ERR_NULL;
  const bool need_q = max_seqlen_q > 0 && total_q > 0, need_k = max_seqlen_k > 0;
  if ((need_k && (k == nullptr || v == nullptr || dk == nullptr || dv == nullptr)) ||
      (need_q && (q == nullptr || o == nullptr || lse == nullptr || dout == nullptr ||
                  dq == nullptr || workspace == nullptr)))
    return ATTN_ERR_NULL;
  if ((need_q && (!aligned16(q) || !aligned16(o) || !aligned16(dout) || !aligned16(dq) ||
                  !aligned16(workspace) || (reinterpret_cast<uintptr_t>(lse) % 4) != 0)) ||
      (need_k && (!aligned16(k) || !aligned16(v) || !aligned16(dk) || !aligned16(dv))))
    return ATTN_ERR_ALIGN;
  const long rows = (long)total_q * Hq;
  if (rows > INT_MAX) return ATTN_ERR_TOO_LARGE;
  hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  BwdParams p{};
  p.q = static_cast<const __bf16*>(q);
  p.k = static_cast<const __bf16*>(k);
  p.v = static_cast<const __bf16*>(v);
  p.dout = static_cast<const __bf16*>(dout);
  float* lse2 = static_cast<float*>(workspace);
  p.lse2 = lse2;
  p.delta = lse2 + rows;
  p.dq = static_cast<__bf16*>(dq);
  p.dk = static_cast<__bf16*>(dk);
  p.dv = static_cast<__bf16*>(dv);
  p.cu_q = cu_seqlens_q;
  p.cu_k = cu_seqlens_k;
  p.seq_order = seq_order;
  p.B = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.Nq = max_seqlen_q;
  p.Nk = max_seqlen_k;
  p.Tq = total_q;
  p.scale = scale;
  p.c = static_cast<float>(static_cast<double>(scale) * 1.4426950408889634);
  return launch_backward(d, p, static_cast<const __bf16*>(o), lse, 1, total_q,
                         cu_seqlens_q + num_seqs, need_q, need_k, causal != 0, st);
}

extern "C" int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o,
                               const float* lse, const void* dout, void* dq, void* dk, void* dv,
                               void* workspace, const int32_t* cu_seqlens_q,
                               const int32_t* cu_seqlens_k, int num_seqs, int total_q, int Hq,
                               int Hkv, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                               int causal, void* stream) {
  return attn_bwd_varlen_ordered(q, k, v, o, lse, dout, dq, dk, dv, workspace, cu_seqlens_q,
                                 cu_seqlens_k, num_seqs, total_q, Hq, Hkv, max_seqlen_q,
                                 max_seqlen_k, d, scale, causal, nullptr, stream);
}
