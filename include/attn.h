/*
 * attn.h - C ABI of the MI355X (gfx950) fused exact-attention forward.
 *
 * The operation.  For every batch element b, query head h and query row i:
 *
 *     O[b,i,h,:] = sum_j P_ij V[b,j,h/G,:],   P_ij = exp(s_ij - LSE_i) for visible j,
 *     s_ij       = scale * <Q[b,i,h,:], K[b,j,h/G,:]>,
 *     LSE_i      = ln sum_{visible j} exp(s_ij)                     (natural log)
 *
 * i.e. O = softmax(scale * Q K^T) V taken row-wise over the visible keys, with
 * the per-row log-sum-exp as a second output.  This is the problem statement of
 * "FlashAttention-4: Algorithm and Kernel Pipelining Co-Design for Asymmetric
 * Hardware Scaling" (papercache summary), section 2.1, and of "059 ·
 * FlashAttention" (wq-win), section 2; the log-sum-exp is the softmax
 * normaliser the forward saves for the backward (FlashAttention notes
 * (xwysyy), "Recomputation").  The N x N score and probability matrices are
 * never written to memory: the kernel walks query blocks x key blocks with the
 * online-softmax running maximum, running sum and unnormalised accumulator
 * (FlashAttention V1 到 V4 (chengxuchu), section 3.4.1).
 *
 * Visibility.  Key j is visible to query i iff
 *     (causal == 0 || j <= i)  &&  j < nk_b,
 * where nk_b = Nk, or seqlens_k[b] clamped to [0, Nk] when seqlens_k is given.
 * The causal mask is top-left aligned (query i sees keys 0..i) also when
 * Nq != Nk.  A row with no visible key gets O = 0 and LSE = -inf.
 *
 * Grouped-query heads: query head h reads key/value head h / G, G = Hq / Hkv.
 *
 * Types and layouts (all row-major, innermost dimension contiguous, no gaps):
 *     q, o : bf16 [B, Nq, Hq, d]        k, v : bf16 [B, Nk, Hkv, d]
 *     lse  : fp32 [B, Hq, Nq]
 *   packed (varlen) form:
 *     q, o : bf16 [Tq, Hq, d]           k, v : bf16 [Tk, Hkv, d]
 *     lse  : fp32 [Hq, Tq],             Tq = cu_seqlens_q[num_seqs]
 * d must be 64 or 128 (forward and backward).  q, k, v and o must be
 * 16-byte aligned; lse 4-byte.
 * O is rounded to bf16 (round-to-nearest-even); LSE stays fp32.
 *
 * Memory and ownership.  Every pointer (q, k, v, o, lse, seqlens_k,
 * cu_seqlens_*, and the backward's dout, dq, dk, dv, workspace) is a DEVICE
 * pointer owned by the caller.  The library allocates nothing, keeps no
 * state besides a thread-local copy of the last HIP error, and is
 * re-entrant.  o and lse must not overlap the inputs or each
 * other.  All calls are asynchronous on `stream` (a hipStream_t; NULL means
 * the default stream): they return after the launch and never synchronise.
 *
 * Errors.  Arguments are validated on the host before any HIP call; a
 * non-zero return code means nothing was launched (except ATTN_ERR_LAUNCH,
 * whose HIP code is kept for attn_last_hip_error()).  Device-resident values
 * (seqlens_k, cu_seqlens_*) are not read on the host: seqlens_k entries are
 * clamped to [0, Nk] in the kernel; cu_seqlens_* must be non-decreasing,
 * start at 0 and stay within the packed buffers, and every sequence length
 * must be at most the max_seqlen passed with it (rows past max_seqlen_q are
 * not computed; keys past max_seqlen_k are not read).
 */
#ifndef EXACT_ATTENTION_18_AMD_ATTN_H
#define EXACT_ATTENTION_18_AMD_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum attn_status {
  ATTN_OK = 0,
  ATTN_ERR_NULL = -1,      /* a required pointer is NULL                          */
  ATTN_ERR_HEAD_DIM = -2,  /* d is not 64 or 128                                  */
  ATTN_ERR_HEADS = -3,     /* Hkv < 1, Hq < 1 or Hq % Hkv != 0                     */
  ATTN_ERR_SIZE = -4,      /* negative size, or scale not finite                  */
  ATTN_ERR_LAUNCH = -5,    /* the HIP launch failed (see attn_last_hip_error)     */
  ATTN_ERR_ALIGN = -6,     /* q, k, v or o not 16-byte aligned, lse not 4-byte    */
  ATTN_ERR_TOO_LARGE = -7, /* grid or index range exceeds what the kernel handles */
  ATTN_ERR_SCRATCH = -8    /* attn_bwd_noalloc: more rows than its static scratch  */
};

/*
 * Batched (padded) forward.
 *   q, k, v   : device bf16 inputs, layouts above.
 *   o, lse    : device outputs, written in full (every row of every head).
 *   B, Nq, Nk : batch size, query and key sequence lengths (>= 0).  B == 0 or
 *               Nq == 0 is a no-op returning ATTN_OK.  Nk == 0 gives O = 0,
 *               LSE = -inf.
 *   Hq, Hkv   : query and key/value head counts (Hq % Hkv == 0).
 *   d         : head dimension, 64 or 128.
 *   scale     : any finite value (the workloads use 1/sqrt(d)).  A negative
 *               scale is computed exactly as scale' = -scale with every query
 *               element negated (a sign flip is exact in bf16); scale == 0
 *               makes every visible key equally likely (O = mean of the
 *               visible V rows, LSE = ln(#visible)).
 *   causal    : non-zero for the causal mask.
 *   seqlens_k : NULL, or device int32 [B] of valid key counts per batch
 *               element (key padding); shared by all heads.
 *   stream    : hipStream_t to launch on (NULL: default stream).
 * Returns an attn_status (ATTN_ERR_TOO_LARGE when B * Nq or B * Nk exceeds
 * 2^31 - 1; element offsets are 64-bit, so arrays may exceed 4 GiB).
 */
int attn_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
             void* stream);

/*
 * Batched forward with different head dimensions for the scores and the
 * values: q, k are bf16 [.., d_qk], v and o bf16 [.., d_v]; everything else
 * (masks, GQA, seqlens_k, lse, errors) as for attn_fwd.  Supported pairs:
 * d_qk == d_v (then this is attn_fwd), and (d_qk, d_v) = (192, 128), the
 * asymmetric shape of the FlashAttention-4 benchmarks ("FlashAttention-4"
 * (papercache summary), experimental setup: head dimensions 64, 128 and
 * (192, 128)).  Other pairs return ATTN_ERR_HEAD_DIM.
 */
int attn_fwd_dims(const void* q, const void* k, const void* v, void* o, float* lse, int B, int Hq,
                  int Hkv, int Nq, int Nk, int d_qk, int d_v, float scale, int causal,
                  const int32_t* seqlens_k, void* stream);

/*
 * Block-sparse batched forward (FlashAttention notes (xwysyy),
 * "Block-Sparse FlashAttention": S = scale Q K^T with the positions of zero
 * blocks of a block mask set to -inf, then P = softmax(S), O = P V).  The
 * block mask is applied on top of the causal and padding masks; everything
 * else (layouts, GQA, seqlens_k, lse, errors) is as for attn_fwd.
 *   block_mask : device uint8 [mask_heads, ceil(Nq/128), ceil(Nk/128)];
 *                entry [h][i][j] != 0 lets query rows 128i..128i+127 of head h
 *                see keys 128j..128j+127.  Shared by every batch element.
 *   mask_heads : 1 (one mask for every head) or Hq (one per query head);
 *                otherwise ATTN_ERR_HEADS.
 * d must be 128 (ATTN_ERR_HEAD_DIM otherwise) and Nk <= 262144
 * (ATTN_ERR_TOO_LARGE otherwise).  Key tiles of zero blocks are neither
 * loaded nor computed.  A row whose visible set is empty gets O = 0 and
 * LSE = -inf.
 */
int attn_fwd_blocksparse(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                         int Hq, int Hkv, int Nq, int Nk, int d, float scale, int causal,
                         const int32_t* seqlens_k, const uint8_t* block_mask, int mask_heads,
                         void* stream);

/*
 * Packed variable-length forward: num_seqs sequences stored back to back.
 * Sequence z owns query rows cu_seqlens_q[z] .. cu_seqlens_q[z+1]-1 and keys
 * cu_seqlens_k[z] .. cu_seqlens_k[z+1]-1; indices are local to the sequence
 * for the causal rule.  cu_seqlens_q / cu_seqlens_k are device int32
 * [num_seqs + 1].  max_seqlen_q / max_seqlen_k bound every sequence's length.
 * Query rows that belong to no sequence are not written.  The packed layout
 * is the batched one with the batch and sequence dimensions flattened
 * (FlashAttention notes (xwysyy), code-structure overview, the "unpadded"
 * interface; FlashAttention-4 (papercache summary), section 3.3, varlen
 * metadata held on the device).  Workgroups take the sequences in index
 * order; scale, causal, errors and ownership are as for attn_fwd.
 */
int attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs,
                    int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                    int causal, void* stream);

/*
 * attn_fwd_varlen with the sequences scheduled in a given order: the
 * virtual-to-actual batch index map of FlashAttention-4 (papercache summary),
 * section 3.3, that the LPT preprocessing kernel (attn_varlen_plan) writes
 * and the attention kernel reads back.
 *   seq_order : NULL (then this is attn_fwd_varlen) or a device int32
 *               [num_seqs] permutation, as attn_varlen_plan writes it;
 *               workgroups take sequence seq_order[v] v-th.  Out-of-range
 *               entries are clamped, never read out of bounds.
 * Every other argument is as for attn_fwd_varlen.  The order changes only
 * the schedule, never a result: outputs are bitwise those of attn_fwd_varlen.
 */
int attn_fwd_varlen_ordered(const void* q, const void* k, const void* v, void* o, float* lse,
                            const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                            int num_seqs, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k,
                            int d, float scale, int causal, const int32_t* seq_order,
                            void* stream);

/*
 * Longest-processing-time-first order of the sequences of a packed batch
 * ("FlashAttention-4" (papercache summary), section 3.3, LPT for variable
 * sequence lengths: a preprocessing kernel sorts the batches by the running
 * time of their longest work tile and writes a virtual-to-actual batch index
 * map that the attention kernel reads back; the map can be cached).
 *   cu_seqlens_q, cu_seqlens_k : device int32 [num_seqs + 1], as for
 *               attn_fwd_varlen.
 *   max_seqlen_q, max_seqlen_k : the same bounds attn_fwd_varlen receives.
 *   causal    : the mask the forward will use (it changes the sort key).
 *   seq_order : device int32 [num_seqs], written: seq_order[v] is the
 *               sequence the forward processes v-th.  It is a permutation of
 *               0 .. num_seqs-1 in non-increasing order of the key
 *               ceil(w / 64), w = min(lq, lk) keys under the causal mask,
 *               lk otherwise (lq, lk: the sequence's lengths clamped to the
 *               max_seqlen bounds); the order among equal keys is
 *               unspecified and does not change any output of the forward.
 * Pass seq_order to attn_fwd_varlen_ordered or attn_bwd_varlen_ordered.
 * num_seqs == 0 is a no-op.  Asynchronous on stream; allocates nothing.
 * Returns an attn_status (ATTN_ERR_NULL for a NULL pointer with num_seqs > 0,
 * ATTN_ERR_SIZE for negative sizes).
 */
int attn_varlen_plan(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs,
                     int max_seqlen_q, int max_seqlen_k, int causal, int32_t* seq_order,
                     void* stream);

/*
 * Backward pass of the batched forward above (FlashAttention-4 (papercache
 * summary), section 2.1, the backward equations; "059 · FlashAttention"
 * (wq-win), section 3, recomputation from the saved row statistics):
 *     dV = P^T dO,  dP = dO V^T,  dS = (diag(p) - p p^T) dp row-wise,
 *     dQ = scale dS K,  dK = scale dS^T Q,
 * where P = exp(S - LSE) is rebuilt from the forward's LSE.  The gradient of a
 * KV head sums over its G = Hq / Hkv query heads.  Masks, GQA map, layouts
 * and `seqlens_k` are those of attn_fwd; keys past seqlens_k[b] get zero
 * gradient.
 *   q, k, v, seqlens_k, scale, causal : exactly as passed to attn_fwd (any
 *               finite scale).
 *   o, lse    : the forward's outputs for these inputs (bf16 [B,Nq,Hq,d] and
 *               fp32 [B,Hq,Nq], natural log).
 *   dout      : bf16 [B,Nq,Hq,d], gradient of the loss with respect to O.
 *   dq        : bf16 [B,Nq,Hq,d], written in full.
 *   dk, dv    : bf16 [B,Nk,Hkv,d], written in full (every key of every KV head).
 *   workspace : device memory of attn_bwd_workspace_size(B, Hq, Nq) bytes,
 *               16-byte aligned, owned by the caller; its contents on entry do
 *               not matter and on return are unspecified.  Calls that overlap
 *               on the GPU need separate workspaces.
 *   d         : 64 or 128.
 * Results are deterministic: every dQ row is summed inside one workgroup and
 * every dK / dV row likewise, with no atomic adds.  Asynchronous on stream;
 * allocates nothing.  Returns an attn_status (ATTN_ERR_HEAD_DIM for d not 64 or 128;
 * ATTN_ERR_NULL / ATTN_ERR_ALIGN as for attn_fwd, including the workspace;
 * ATTN_ERR_TOO_LARGE when B * Nq * Hq or B * Nk * Hkv exceeds 2^31 - 1).
 * B == 0, or Nq == 0 and Nk == 0, is a no-op.
 */
int attn_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
             const void* dout, void* dq, void* dk, void* dv, void* workspace, int B, int Hq,
             int Hkv, int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
             void* stream);

/*
 * Backward pass of the packed variable-length forward (attn_fwd_varlen):
 * the same equations as attn_bwd, per sequence, with the sequences stored
 * back to back as that forward describes (FlashAttention notes (xwysyy),
 * code-structure overview, the "unpadded" interface).
 *   q, k, v, cu_seqlens_q, cu_seqlens_k, num_seqs, max_seqlen_q,
 *   max_seqlen_k, scale, causal : as passed to attn_fwd_varlen.
 *   total_q   : rows of q, o, dout and dq (at least cu_seqlens_q[num_seqs]).
 *   o, lse    : that forward's outputs: bf16 [total_q, Hq, d] and fp32 LSE
 *               rows of cu_seqlens_q[num_seqs] entries per head, as it writes
 *               them.
 *   dout, dq  : bf16 [total_q, Hq, d]; dq rows of the sequences are written.
 *   dk, dv    : bf16 [Tk, Hkv, d]; rows of the sequences' keys are written
 *               (zero for keys that no query sees).  Rows outside every
 *               sequence are not touched.
 *   workspace : attn_bwd_workspace_size(1, Hq, total_q) bytes, as for
 *               attn_bwd.
 *   d         : 64 or 128.
 * Deterministic, asynchronous on stream, allocates nothing.  Returns an
 * attn_status as attn_bwd does (ATTN_ERR_NULL also for NULL cu_seqlens).
 * num_seqs == 0, or both max_seqlen bounds 0, is a no-op.
 */
int attn_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, void* workspace,
                    const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, int num_seqs,
                    int total_q, int Hq, int Hkv, int max_seqlen_q, int max_seqlen_k, int d,
                    float scale, int causal, void* stream);

/*
 * attn_bwd_varlen with the sequences scheduled in the order seq_order (NULL,
 * or the device int32 [num_seqs] permutation attn_varlen_plan writes; the
 * batch index map of FlashAttention-4 (papercache summary), section 3.3).
 * The order changes only the schedule: results are bitwise those of
 * attn_bwd_varlen.  Every other argument is as for attn_bwd_varlen.
 */
int attn_bwd_varlen_ordered(const void* q, const void* k, const void* v, const void* o,
                            const float* lse, const void* dout, void* dq, void* dk, void* dv,
                            void* workspace, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int num_seqs, int total_q, int Hq,
                            int Hkv, int max_seqlen_q, int max_seqlen_k, int d, float scale,
                            int causal, const int32_t* seq_order, void* stream);

/*
 * attn_bwd without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The LSE * log2(e) and D rows that
 * attn_bwd keeps in the caller's workspace live instead in a static device
 * array of 32 MiB, of which each GPU the library runs on holds its own copy
 * until the process ends.  This call allocates nothing (no hipMalloc, no
 * allocating library routine); its first call on a device looks up the
 * array's device address there (hipGetSymbolAddress).
 *   Arguments, results and errors: as for attn_bwd (without workspace), plus
 *   ATTN_ERR_SCRATCH when B * Hq * Nq > 4194304 (nothing is launched).
 * Every call on one GPU shares that GPU's array: calls that overlap on a GPU
 * (other streams, other host threads) race and must be serialised by the
 * caller.  Each call writes every array entry it reads before reading it, so
 * what an earlier call left there never reaches a result.
 */
int attn_bwd_noalloc(const void* q, const void* k, const void* v, const void* o, const float* lse,
                     const void* dout, void* dq, void* dk, void* dv, int B, int Hq, int Hkv,
                     int Nq, int Nk, int d, float scale, int causal, const int32_t* seqlens_k,
                     void* stream);

/* Bytes of workspace attn_bwd needs: two fp32 per (batch, query head, query
 * row); 0 when any argument is <= 0. */
size_t attn_bwd_workspace_size(int B, int Hq, int Nq);

/* Static text for an attn_status code (never NULL). */
const char* attn_strerror(int status);

/*
 * Matrix-core rate probe (a measurement aid; it computes nothing of the
 * attention).  The roofline analysis of FlashAttention-4 (papercache
 * summary), section 3.1.1, prices the attention tile in cycles of the matrix
 * core; this call measures what that unit sustains on the device under a full
 * grid, with either MFMA shape the forward uses (v_mfma_f32_32x32x16_bf16:
 * the d = 64 and (192, 128) kernels; v_mfma_f32_16x16x32_bf16: the d = 128
 * kernel) and no other work, so the forward's rate can be compared
 * with it as well as with the published peak.  The clock drops under
 * matrix-core load by an amount that depends on the operand bits, hence the
 * caller-supplied operands.
 *   operands   : device bf16 [8][64][8], 16-byte aligned: for each of 4 A and
 *                then 4 B operands, lane l's 8 elements.
 *   shape      : 32 (v_mfma_f32_32x32x16_bf16: 16 MFMAs per iteration into
 *                8 accumulators) or 16 (v_mfma_f32_16x16x32_bf16: 32 MFMAs
 *                per iteration into 16 accumulators); either way 16 * 32768
 *                FLOP per wave and iteration.
 *   iters      : loop iterations per wave, >= 1.  FLOP per launch =
 *                workgroups * 8 waves * iters * 16 * 32768.
 *   workgroups : >= 1; 512 threads each (8 waves, two per SIMD), one resident
 *                per CU (each reserves 84 KB of LDS), as the forward's; pass
 *                the CU count to run every CU once.
 *   sink       : device fp32 [workgroups * 512], written (keeps the work live).
 *                With every operand element 1.0 each value is 4096 * iters.
 *   clocks     : device uint64 [workgroups * 8][2], written: per wave the
 *                shader-clock ticks (s_memtime) and the constant 100 MHz
 *                real-time ticks (s_memrealtime) across its loop, whose
 *                ratio gives the shader clock.
 * Returns ATTN_ERR_NULL, ATTN_ERR_SIZE (shape not 32 or 16, iters or
 * workgroups < 1), ATTN_ERR_ALIGN, ATTN_ERR_TOO_LARGE or ATTN_ERR_LAUNCH;
 * asynchronous on stream like every other call.
 */
int attn_probe_mfma(const void* operands, int shape, int iters, int workgroups, float* sink,
                    uint64_t* clocks, void* stream);

/*
 * Softmax issue probe (a measurement aid; it computes nothing of the
 * attention).  FlashAttention-4 (papercache summary), section 3.1.3,
 * evaluates part of each row's exp2 as a polynomial on the FMA units because
 * its exponential unit limits the softmax.  This call prices that choice on
 * this device: in each 512-thread workgroup (one per CU, as the forward's),
 * waves 0-3 stream v_mfma_f32_32x32x16_bf16 (mfma_on = 1) or idle (0), and waves
 * 4-7, one beside each of them on its SIMD, run the forward's softmax
 * instruction mix on 32 elements per lane and iteration (FMA, exp2, running
 * sum, v_max3, bf16 packing).  exp_kind: 0 = those waves idle,
 * 1 = v_exp_f32, 2 = a degree-3 polynomial exp2 on the FMA pipe (Cody-Waite
 * split, own minimax coefficients), 3 = the polynomial on 8 of the 32
 * elements and v_exp_f32 on the rest.  Every wave runs until budget_us
 * microseconds of real time have passed.
 *   operands  : device bf16 [8][64][8], 16-byte aligned, as attn_probe_mfma.
 *   values    : device fp32 [64 * 32], written when exp_kind != 0: lane l's
 *               exponentials of x_i = (l + 64 i) / 256 - 8, i = 0..31, by
 *               the kind's method (for an accuracy check).
 *   stats     : device uint64 [workgroups * 8][4], written per wave:
 *               iterations (16 MFMAs, or 32 elements per lane), shader-clock
 *               ticks (s_memtime), 100 MHz ticks (s_memrealtime), and a
 *               checksum's bits (keeps the work live).  Idle waves write 0.
 *   budget_us : 1 .. 10000000.   workgroups : >= 1.
 * Returns ATTN_ERR_NULL, ATTN_ERR_SIZE, ATTN_ERR_ALIGN, ATTN_ERR_TOO_LARGE
 * or ATTN_ERR_LAUNCH; asynchronous on stream.
 */
int attn_probe_softmax_issue(const void* operands, int mfma_on, int exp_kind, int budget_us,
                             int workgroups, float* values, uint64_t* stats, void* stream);

/*
 * Workgroup placement probe (a measurement aid; it computes nothing of the
 * attention).  The grid order of the forward keeps the key/value tiles of a
 * (batch, KV head) unit in one XCD's L2 by dealing units round-robin to the
 * XCDs, which the heads-in-L2-sections scheduling of FlashAttention-4
 * (papercache summary), section 3.3, calls for; that rests on the dispatcher
 * placing workgroup w on XCD w % 8.  This call records where each workgroup of
 * a grid of 512-thread workgroups (the forward's size, one per CU) runs.
 *   workgroups : >= 1.
 *   ids        : device int32 [workgroups][2], 8-byte aligned, written:
 *                ids[w][0] = the XCD (hardware register XCC_ID, 0..7) and
 *                ids[w][1] = the raw HW_ID register of the workgroup's first
 *                wave (shader engine, CU, SIMD, wave slot).
 * Returns ATTN_ERR_NULL, ATTN_ERR_SIZE, ATTN_ERR_ALIGN, ATTN_ERR_TOO_LARGE or
 * ATTN_ERR_LAUNCH; asynchronous on stream.
 */
int attn_probe_xcd(int workgroups, int32_t* ids, void* stream);

/* hipError_t of the last failed launch on this thread (0 if none). */
int attn_last_hip_error(void);

/* Library version, e.g. "0.1.0". */
const char* attn_version(void);

#ifdef __cplusplus
}
#endif

#endif /* EXACT_ATTENTION_18_AMD_ATTN_H */
