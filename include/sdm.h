/* sdm.h -- C ABI of the Sparse Delta Memory (SDM) step library (libsdm.so),
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The step (pages "Riepilogo Tecnico: Sparse Delta Memory (SDM)",
 * gist.science/it/paper/2607.07386, and its Japanese twin
 * gist.science/ja/paper/2607.07386; section "Meccanismo Core" items 1-4 and
 * section "Stato Iniziale Appreso"):
 *   - the state is an explicit table M of N = n*n slots, each a row of d_v
 *     values, one table per (batch b, head h);
 *   - a key and a query are each split in two halves (x1, x2) of length n;
 *     slot f = a*n + b scores x1[a] + x2[b]; the top-K slots are found with
 *     topk(x1 (+) x2) = topk(topk(x1) (+) topk(x2)) without forming all N
 *     scores (K = W for writes, K = R for reads);
 *   - the selected write rows get the gated delta update
 *       Mt[i] = alpha_t * M[i];  M[i] = Mt[i] + beta_t * k_i * (v_t - Mt[i]),
 *     all other rows stay as they are;
 *   - the output is the weighted sum of the selected read rows;
 *   - every sequence starts from a learned initial table M0.
 * The pages do not say how the weights k_i and the read weights are formed;
 * this library uses softmax over the selected summed scores, and reads after
 * the step's write.
 *
 * Conventions for every call
 *   - Every buffer pointer is a DEVICE pointer to caller-owned memory,
 *     contiguous, row-major, in the layout stated per argument.  The library
 *     allocates nothing, keeps no pointer after the call returns, and only
 *     writes the documented outputs (and M, updated in place).
 *   - `stream` is a hipStream_t (passed as void*; NULL = the null stream).
 *     Work is enqueued asynchronously in call order; nothing synchronises the
 *     host unless the environment variable SDM_DEBUG_SYNC=1 is set, which
 *     makes each call wait for its kernels and report asynchronous errors.
 *   - All arguments are validated before any launch.  Return values:
 *       SDM_OK (0)               success (work enqueued);
 *       SDM_ERR_INVALID (1)      bad argument (null pointer, size out of
 *                                range, misaligned pointer); nothing enqueued;
 *       SDM_ERR_UNSUPPORTED (2)  a shape outside the compiled set; nothing
 *                                enqueued (there is no fallback path);
 *       SDM_ERR_HIP (3)          the HIP runtime reported an error.
 *     A human-readable reason for the last non-OK return on the calling
 *     thread is available from sdm_last_error().  Nothing throws or aborts.
 *   - Supported shapes: n in 1..64 or n in {128, 256, 512, 1024, 2048};
 *     1 <= K, W, R <= min(n, 64); d_v in {16, 32, 64, 128, 256};
 *     state dtype SDM_F32 or SDM_BF16 (bf16 state uses fp32 arithmetic and
 *     rounds to nearest even on store), or SDM_FP8 for sdm_state_init and
 *     sdm_scan with d_v >= 32: OCP FP8 E4M3 codes ("e4m3fn", bias 7, largest
 *     finite 448), fp32 arithmetic, rounded to nearest even on store; the
 *     write is then evaluated in a fixed binary32 order with no contraction
 *     -- Mt = alpha*M, d = v - Mt, M = fma(beta*k, d, Mt) -- so the stored
 *     codes are a function of the binary32 inputs alone.  Pointers to M, M0 and v must be
 *     16-byte aligned; sub-score pointers must be 16-byte aligned when
 *     n >= 256 and 4-byte aligned otherwise.
 *   - Size limits per call (a kernel launch counts its work-items in 32 bits):
 *     at most 2^20 memories (B*H) for every call that walks memories, and at
 *     most 2^26 - 4 selection units (sdm_select, sdm_select_backward) or
 *     memory-steps B*H*T (sdm_scan_backward), and for the scans at most 2^32
 *     steps T and 2^40 memory-steps B*H*T; larger work is split by the
 *     caller into several calls.  Beyond them a call returns
 *     SDM_ERR_UNSUPPORTED before launching anything.
 *   - Calls on different streams are independent as long as they do not
 *     share an output buffer (including M).
 */
#ifndef SDM_H
#define SDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { SDM_OK = 0, SDM_ERR_INVALID = 1, SDM_ERR_UNSUPPORTED = 2, SDM_ERR_HIP = 3 };
enum { SDM_F32 = 0, SDM_BF16 = 1, SDM_FP8 = 2 };

/* Token projections in front of the step ("Meccanismo Core", item 2: the
 * projected key k' and query q' are each split in two halves; section
 * "Design IsoFLOP": the projections are sized like the baseline's).  For
 * token m = b*T + t and head h, y = Wt[h] x_m (P = 4n + d_v + 2 rows per
 * head), on the matrix cores: bf16 inputs, fp32 accumulation.
 *   X      [B*T, d_model] bf16 bits in (row-major, 16-byte aligned).
 *   Wt     [H, P, d_model] bf16 bits in (16-byte aligned): per head the rows
 *          giving, in order, s1 (n rows), s2 (n), q1 (n), q2 (n), v (d_v),
 *          the alpha pre-activation and the beta pre-activation.
 *   s1, s2, q1, q2  [B, H, T, n] fp32 out: the write key halves and the
 *          read query halves (the layout sdm_select takes, units = B*H*T).
 *   v      [B, H, T, d_v] fp32 out.
 *   alpha, beta  [B, H, T] fp32 out: 1 / (1 + exp(-y)) of the two gate rows.
 * Each y is a binary32 sum of the d_model exact bf16 products, in an
 * unspecified order: |y - exact| <= (d_model - 1) * 2^-23 * sum |x_i w_i|
 * (unit roundoff 2^-23 covers any rounding of the additions inside the
 * matrix unit), plus a few ulps of expf and division for the gates.  Sizes: d_model a multiple of 64 in [64, 65536];
 * n, d_v >= 1; H*P < 2^31; at most 2^24 - 1 tiles of 256 tokens x 256
 * columns per call.  B*T = 0 is a valid no-op (every array may then be
 * NULL).  Output pointers must be 4-byte aligned. */
int sdm_project(const uint16_t* X, const uint16_t* Wt, int B, int T, int d_model, int H, int n,
                int d_v, float* s1, float* s2, float* q1, float* q2, float* v, float* alpha,
                float* beta, void* stream);

/* Product-key top-K selection with softmax weights ("Meccanismo Core",
 * item 2), for `units` independent (key or query) half pairs.
 *   x1, x2  [units, n] fp32 half sub-scores (all values finite, and every
 *           sum x1[a] + x2[b] finite, so the weights are defined).
 *   idx     [units, K] int32 out: flat slots f = a*n + b, ordered by
 *           (score descending, f ascending).  Stage 1 keeps, per half, the K
 *           indices of largest value (lower index first on equal values);
 *           stage 2 ranks the K*K binary32 sums x1[a] + x2[b] the same way.
 *           -0.0 compares equal to +0.0.
 *   score   [units, K] fp32 out: the selected sums, or NULL.
 *   weight  [units, K] fp32 out: exp(score_j - score_0) / sum_l exp(...).
 * units = 0 is a valid no-op (x1, x2, idx, score and weight may then be NULL). */
int sdm_select(const float* x1, const float* x2, int64_t units, int n, int K, int32_t* idx,
               float* score, float* weight, void* stream);

/* Learned initial state ("Stato Iniziale Appreso"): M[b,h] = M0[h] for every
 * batch row b.
 *   M   [B, H, N, d_v] out, fp32 (dtype SDM_F32), bf16 bits (SDM_BF16) or
 *       E4M3 codes (SDM_FP8), the last two rounded to nearest even.
 *   M0  [H, N, d_v] fp32 in. */
int sdm_state_init(void* M, int dtype, const float* M0, int B, int H, int64_t N, int d_v,
                   void* stream);

/* T sequential steps of the gated delta write and the sparse read
 * ("Meccanismo Core", items 3 and 4) on every (b,h) memory, in place.
 *   M       [B, H, N, d_v] state (fp32, bf16 bits or fp8 E4M3 codes),
 *           updated in place.
 *   widx    [B, H, T, W] int32 write rows of each step (as sdm_select
 *           returns them); the W rows of one step must be distinct.
 *   wk      [B, H, T, W] fp32 write weights k.
 *   ridx    [B, H, T, R] int32 read rows;  rw [B, H, T, R] fp32 read weights.
 *   v       [B, H, T, d_v] fp32 values;  alpha, beta [B, H, T] fp32 gates.
 *   out     [B, H, T, d_v] fp32 out: o_t = sum_j rw_j * M_t[ridx_j], read
 *           from the state after step t's write (as stored, i.e. after the
 *           bf16 or fp8 rounding).
 * Per step and row: Mt = alpha*M; M = Mt + (beta*k)*(v - Mt), in fp32.
 * Rows not selected for writing are never touched.  Row indices outside
 * [0, N) are skipped (no access; a skipped read row contributes 0); repeated
 * write rows within one step leave those rows unspecified.  T = 0 is a
 * valid no-op (the per-step arrays may then be NULL).  The caller may split a sequence into consecutive calls over
 * consecutive time ranges; the result is identical. */
int sdm_scan(void* M, int dtype, int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
             const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
             const float* v, const float* alpha, const float* beta, float* out, void* stream);

/* ---- Planned scan (fp32 state): the steps of sdm_scan ("Meccanismo Core",
 * items 3 and 4) in two calls, for workloads with few memories (long
 * sequences on a handful of heads).  The first call turns the step indices
 * into per-shard compacted row lists in a caller workspace; the second runs
 * the steps from those lists.  The rows of a memory are split between S row
 * shards (S = 1, 2 or 8, chosen from B*H and d_v so the workgroups fill the
 * GPU), each moved in whole 128-byte row pieces (32 columns).
 *
 * Results: M equal to sdm_scan's bit for bit (the same fp32 update of the
 * same rows in the same step order); out equal to it up to the order of
 * the read's fp32 additions (per shard in list order, then the shards in a
 * fixed order), so it is deterministic and the same for any split of the
 * sequence into consecutive calls.  Index, weight and gate semantics are
 * sdm_scan's (rows outside [0, N) are skipped; repeated write rows within
 * one step leave those rows unspecified). */

/* Bytes of workspace for these sizes (0 if they are not supported: B, H < 1,
 * B*H > 2^20, T < 0 or T > 2^20, d_v not one of 32, 64, 128, 256).  The workspace holds the lists of
 * every step and, with S > 1, one fp32 partial output per shard; it grows
 * with B*H*T, so long sequences are planned and run in consecutive calls of
 * a bounded T (16384 steps of 16 memories at d_v = 128: about 3.8 GB). */
size_t sdm_scan_plan_workspace_size(int B, int H, int d_v, int64_t T);

/* Plan T steps (T <= 2^20 per call).
 *   widx, wk, ridx, rw  as for sdm_scan; W, R in [1, 64].
 *   workspace  device buffer of at least sdm_scan_plan_workspace_size bytes,
 *              256-byte aligned, written by this call (no clearing needed).
 * T = 0 is a no-op (the arrays may then be NULL). */
int sdm_scan_plan(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                  const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
                  void* workspace, size_t workspace_bytes, void* stream);

/* Run the T steps that sdm_scan_plan wrote into workspace, on the fp32
 * state M [B, H, N, d_v] in place; v, alpha, beta and out as for sdm_scan
 * (out 16-byte aligned).  B, H, N, d_v and T must be those of the plan call
 * (rows at or past N are skipped, so a mismatch gives wrong values but never
 * an access outside M).  The workspace's partial outputs are overwritten. */
int sdm_scan_planned(void* M, int B, int H, int64_t N, int d_v, int64_t T, const float* v,
                     const float* alpha, const float* beta, float* out, void* workspace,
                     size_t workspace_bytes, void* stream);

/* One single-token step for every (b,h): both selections, the write and the
 * read, fused in one kernel (the recurrent inference form; page "Riepilogo
 * Tecnico: Sparse Delta Memory (SDM)", section "Significato e
 * Rivendicazioni", constant state and compute per token).
 *   M        [B, H, n*n, d_v] state, updated in place.
 *   s1, s2   [B, H, n] write half sub-scores;  q1, q2 [B, H, n] read halves.
 *   v        [B, H, d_v];  alpha, beta [B, H].
 *   out      [B, H, d_v] fp32 out.
 *   widx     [B, H, W] int32 out (selected write rows), or NULL.
 *   ridx     [B, H, R] int32 out (selected read rows), or NULL.
 * Equal to sdm_select twice followed by sdm_scan with T = 1. */
int sdm_step_decode(void* M, int dtype, int B, int H, int n, int d_v, int W, int R,
                    const float* s1, const float* s2, const float* q1, const float* q2,
                    const float* v, const float* alpha, const float* beta, float* out,
                    int32_t* widx, int32_t* ridx, void* stream);

/* ---- Training: the forward with a tape, and the reverse pass.
 * The pages train the layer end to end and learn M0 ("Stato Iniziale
 * Appreso"); these calls give the gradients of the write and read
 * ("Meccanismo Core", items 3 and 4) with the selections held fixed (the
 * chosen slots are piecewise constant in the scores; gradients reach the
 * scores through the selection weights only).  fp32 state only. */

/* sdm_scan (fp32 state) that also keeps, per step, the rows the reverse pass
 * needs, so that the reverse pass never reads or writes the state.
 *   tape  [B, H, T, W + R, d_v] fp32 out: for j < W, tape[b,h,t,j] = the
 *         stored row widx[b,h,t,j] just before step t's write; for j < R,
 *         tape[b,h,t,W+j] = the stored row ridx[b,h,t,j] as step t's read
 *         used it (after the write).  Slots of rows outside [0, N) are not
 *         written.  One memory's tape, T*(W+R)*d_v*4 bytes, must be below
 *         2 GiB (split longer sequences into consecutive calls).
 * Every other argument and output is as for sdm_scan, and the results are
 * identical to it. */
int sdm_scan_train(void* M, int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                   const int32_t* widx, const float* wk, const int32_t* ridx, const float* rw,
                   const float* v, const float* alpha, const float* beta, float* out,
                   float* tape, void* stream);

/* Bytes of workspace sdm_scan_backward needs for these sizes. */
size_t sdm_scan_backward_workspace_size(int B, int H, int d_v, int64_t T, int W, int R);

/* Reverse pass over T steps, t = T-1 .. 0, for every (b,h) memory.  It takes
 * every row value it needs from the tape; the state itself is not an
 * argument (the caller's state keeps whatever the forward left in it).
 *   widx, wk, ridx, rw, v, alpha, beta: the forward's inputs (shapes as for
 *          sdm_scan).  The rows of each step's widx must be distinct, and so
 *          must those of each step's ridx (sdm_select guarantees both).
 *   tape   [B, H, T, W + R, d_v] fp32 in: from sdm_scan_train on the same
 *          inputs.
 *   dout   [B, H, T, d_v] fp32 in: dL/d out.
 *   G      [B, H, N, d_v] fp32 in/out: in, dL/d(state after step T-1) (zeros
 *          when the final state is not used); out, dL/d(state before step 0).
 *   dv     [B, H, T, d_v] fp32 out: dL/dv.
 *   dwk    [B, H, T, W] fp32 out: dL/dk (the write weights).
 *   drw    [B, H, T, R] fp32 out: dL/dr (the read weights).
 *   dalpha, dbeta [B, H, T] fp32 out.
 *   first  NULL (dense mode: G holds dL/dM_T for every row on entry), or
 *          [B, H, T, 2] uint64 from sdm_touch_prepare on the same widx and
 *          ridx (sparse mode: dL/dM_T is taken as zero, and G's contents on
 *          entry do not matter -- each row's first touch in reverse time
 *          starts from zero instead of reading G).  In sparse mode, G holds
 *          dL/dM_0 on exit only for the rows the T steps select (seen);
 *          the other rows keep whatever they held.  Both modes give the same
 *          bits for every selected row of G; the per-step sums (dv, dwk, drw,
 *          dalpha, dbeta) may differ in the last bits (the sparse mode uses
 *          narrower column tiles, so it adds them in another order).  (A chunk of a
 *          sequence whose later chunks' reverse passes already wrote G has a
 *          nonzero dL/dM_T: use the dense mode there.)
 *   workspace  device buffer of at least
 *          sdm_scan_backward_workspace_size(B, H, d_v, T, W, R) bytes,
 *          16-byte aligned; its contents on entry do not matter.
 * Per step, with P the pre-write row of write row f_j and g = G[f_j] after
 * the step's read contributions G[g_l] += r_l * dout_t:
 *   dv_t += beta*k_j*g;  dalpha_t += (1 - beta*k_j)*<g, P>;
 *   dk_j = beta*<g, v_t - alpha*P>;  dbeta_t += k_j*<g, v_t - alpha*P>;
 *   G[f_j] = alpha*(1 - beta*k_j)*g;   dr_l = <dout_t, M_t[g_l]>, with
 * P and M_t[g_l] read from the tape.
 * Arithmetic in fp32; the tile partial sums are added in a fixed order, so
 * results are deterministic.  Sizes as for sdm_scan, plus T < 2^26 and
 * B*H*T <= 2^26 - 4.  T = 0 is a valid no-op (G unchanged; every per-step array
 * and the workspace may then be NULL). */
int sdm_scan_backward(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                      const int32_t* widx, const float* wk, const int32_t* ridx,
                      const float* rw, const float* v, const float* alpha, const float* beta,
                      const float* tape, const float* dout, float* G, float* dv, float* dwk,
                      float* drw, float* dalpha, float* dbeta, const uint64_t* first,
                      void* workspace, size_t workspace_bytes, void* stream);

/* sdm_scan_backward for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): the same reverse pass, with its per-tile partial sums kept in
 * a scratch buffer the library holds on each GPU instead of a caller
 * workspace.  That buffer is 64 MiB (aligned to 256 bytes), set up on a GPU
 * at the first call there and held until the process ends; this call never
 * allocates or frees memory.  Sizes whose workspace
 * (sdm_scan_backward_workspace_size) is above 64 MiB return
 * SDM_ERR_UNSUPPORTED before any launch (use sdm_scan_backward then).  Every
 * call on one GPU uses that GPU's one buffer, whose contents on entry do not
 * matter: calls that overlap in time on one GPU (on different streams or
 * from different threads) race on it and give undefined results, so the
 * caller must order them.  Arguments, outputs and results are otherwise
 * those of sdm_scan_backward, bit for bit. */
int sdm_scan_backward_noalloc(int B, int H, int64_t N, int d_v, int64_t T, int W, int R,
                              const int32_t* widx, const float* wk, const int32_t* ridx,
                              const float* rw, const float* v, const float* alpha,
                              const float* beta, const float* tape, const float* dout, float* G,
                              float* dv, float* dwk, float* drw, float* dalpha, float* dbeta,
                              const uint64_t* first, void* stream);

/* Gradient of the selection weights back to the halves ("Meccanismo Core",
 * item 2: slot f = a*n + b scores x1[a] + x2[b]), selections held fixed.
 *   idx, weight  [units, K] from sdm_select;  dweight [units, K] fp32 in.
 *   dx1, dx2     [units, n] fp32 out: with dsigma_j = w_j*(dw_j - sum_l w_l dw_l),
 *                dx1[a] = sum of dsigma_j over the j with a_j = a (dx2 with
 *                b_j), zero at every half index no selected slot uses.
 * units = 0 is a valid no-op (the arrays may then be NULL). */
int sdm_select_backward(const int32_t* idx, const float* weight, const float* dweight,
                        int64_t units, int n, int K, float* dx1, float* dx2, void* stream);

/* Gradient of the per-sequence copy M[b,h] = M0[h]:
 *   dM0[h] = sum over b = 0, 1, ... of G[b,h].
 *   G [B, H, N, d_v] fp32 in;  dM0 [H, N, d_v] fp32 out (16-byte aligned).
 *   seen  NULL (every row of G counts), or [B, H, ceil(N/32)] uint32 from
 *         sdm_touch_prepare (sparse mode: row r of G[b,h] counts only when
 *         bit r of seen[b,h] is set, and is not read otherwise; the sum is
 *         the same as the dense one with those rows zero). */
int sdm_state_init_backward(const float* G, int B, int H, int64_t N, int d_v,
                            const uint32_t* seen, float* dM0, void* stream);

/* Bookkeeping for the sparse training mode (the method touches only W + R
 * rows per step, "Meccanismo Core" items 3 and 4, so most of the gradient
 * table is never touched by one sequence).
 *   widx [B, H, T, W], ridx [B, H, T, R] int32 in: the forward's selections.
 *   seen  [B, H, ceil(N/32)] uint32 out: bit (r % 32) of word r / 32 is set
 *         when row r is selected (write or read) at any of the T steps.
 *   first [B, H, T, 2] uint64 out: bit j of first[b,h,t,0] is set when
 *         widx[b,h,t,j]'s last selection is step t; first[b,h,t,1] likewise
 *         for ridx.
 * 1 <= W, R <= 64; 1 <= N <= 2^20 (one N-bit table per memory is kept on
 * chip); 0 <= T < 2^26 with T*max(W,R)*4 below 2^31 (T = 0 only clears
 * seen; the index arrays and first may then be NULL).  Indices outside
 * [0, N) are ignored. */
int sdm_touch_prepare(int B, int H, int64_t N, int64_t T, int W, int R, const int32_t* widx,
                      const int32_t* ridx, uint32_t* seen, uint64_t* first, void* stream);

/* Static text for a status code. */
const char* sdm_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* sdm_last_error(void);

/* ABI version of this header (incremented on incompatible change). */
int sdm_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SDM_H */
