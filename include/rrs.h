/*
 * rrs.h -- C ABI of the MI355X (gfx950) Rotated Runtime Smooth A4W4 linear.
 *
 * The layer computes Y = X W for fp16 activations X [M, K] and fp16 weights
 * W [K, N] through the Rotated Runtime Smooth (RRS) recipe:
 *
 *   1. rotate every activation row by the Sylvester Hadamard matrix H_K
 *      (RRS summary page, atlas.scime.ai, "Approach"; normalised Hadamard in
 *      the AGC-OR page, paperpeel.com, Sec. 3.2);
 *   2. reorder the channels by a fixed permutation and divide each group of
 *      G reordered channels by its runtime maximum over the call's tokens
 *      (RRS rebuttal page, paperhub.cn, "Novelty" answer and the reorder
 *      answer Y = X W^T = sum_i X_i W_i^T);
 *   3. quantise each token to symmetric 4-bit codes in [-7, 7] with scale
 *      max|row| / 7 (AGC-OR page, Sec. 3.1 and App. B.1, q_A = 2^(b-1) - 1)
 *      and pack two codes per byte;
 *   4. multiply against offline rotated, reordered, per-output-channel 4-bit
 *      weights, rescaling each K-group's integer partial sum by its group
 *      scale before fp32 accumulation (the smoothing scales stay out of the
 *      weights: RRS summary page, "Approach"; the group-wise scales are
 *      chosen so that the contraction keeps its tiled computation scheme:
 *      RRS rebuttal page, "Novelty" answer).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - All data pointers are DEVICE pointers (hipMalloc / torch CUDA tensors)
 *   unless stated otherwise, each 16-byte aligned (the kernels move data in
 *   16-byte accesses; a misaligned pointer is rejected with RRS_EINVAL). The caller allocates and owns every buffer; the
 *   library never allocates, frees or synchronises, and keeps no global
 *   mutable state.
 * - Every call is asynchronous on the given stream `s` (0 = null stream).
 * - Arguments are validated on the host before any launch; a failing check
 *   returns RRS_EINVAL (or RRS_EUNSUPPORTED for legal but unbuilt shapes) and
 *   launches nothing. A failed launch returns RRS_EHIP.
 * - Shapes: K is a power of two with 64 <= K <= 8192; G is a power of two
 *   with 32 <= G <= K (so G divides K); M >= 1, N >= 1 (M = 0 is accepted by
 *   the entry points that take M and is a no-op).
 * - Layouts: X fp16 [M, K] row-major; W fp16 [K, N] row-major (the
 *   transpose of nn.Linear.weight); Y fp32 [M, N] row-major.
 * - Packed codes: 4-bit sign-magnitude, K in reordered order, 8 codes per
 *   little-endian 32-bit word (4 bytes). With a_j = code 2j and b_j = code
 *   2j+1 of a word, byte j holds |a_j| in bits 0-2, |b_j| in bits 4-6, the
 *   sign of a_j in bit 7 and the sign of b_{(j-1) mod 4} in bit 3. Masking a
 *   word with 0x87878787 then gives its four a codes, and rotating it right
 *   by 4 bits before the same mask its four b codes, each as an fp8 e4m3
 *   byte whose value is exactly code * 2^-9 (a subnormal), which the matrix
 *   cores consume directly. A zero code may carry either sign bit (a
 *   negative value that rounds to 0 keeps its sign); readers take any zero
 *   magnitude as 0. The pages fix no storage layout.
 * - Stored layout of a code matrix (activation codes xq [M rows], prepared
 *   weight codes [N rows], each row K/2 bytes in reordered K order): rows in
 *   pairs, each row cut into 64-byte pieces (128 codes), piece c of rows 2p
 *   and 2p + 1 side by side in one 128-byte line. Byte b of row r lies at
 *     (r / 2) * 2 rs + (b / 64) * 128 + (r % 2) * 64 + b % 64,
 *   rs = K/2 rounded up to 64 (for K = 64, 32 bytes of each piece are
 *   used); rrs_codes_bytes(rows, K) bytes in all (an odd row count leaves
 *   the last pair half used). The GEMMs then read whole 128-byte lines.
 * - Scales are reported in the unnormalised-Hadamard convention:
 *     dx[t] = r_t / 7 with r_t = max_j |Zp[t,j] / S_g(j)|,
 *     S[g]  = max over tokens and the group's channels of |Zp|,
 *     dw[n] = max_j |Wp[j,n]| / 7,
 *   so that Y[t,n] = (1/K) dx[t] dw[n] sum_g S[g] P_g[t,n].
 * - `perm` (int32 [K], device) must be a permutation of 0..K-1 (not checked
 *   on the device): position j of the reordered row takes rotated channel
 *   perm[j].
 * - Signed rotation (the `_signed` entry points): the rotation becomes
 *   Z = X D H_K with D = diag(d), d_j = -1 where bit j of the sign mask
 *   `dsign` is set (uint32 [K/32] words, device, little-endian: bit j % 32
 *   of word j / 32; K >= 64 so at least two words) and +1 elsewhere, and
 *   the weights take H_K D W (the transform family P = D H^T of the AGC-OR
 *   page, Sec. 4.1, with unit channel scaling; the signed online rotation
 *   of its Sec. 4.6). Calibration, weight preparation and the front end of
 *   one layer must use the same mask. `dsign` must not be NULL (use the
 *   plain entry points for D = I).
 * - Non-finite inputs are outside the contract.
 */
#ifndef RRS_H_
#define RRS_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  RRS_OK = 0,
  RRS_EINVAL = -1,       /* bad argument (shape, null pointer, short buffer) */
  RRS_EUNSUPPORTED = -2, /* legal request the library does not serve */
  RRS_EHIP = -3,         /* a HIP launch or runtime call failed */
  RRS_ETOOBIG = -4       /* rrs_linear_noalloc: the call needs more than its fixed scratch */
} rrs_status;

/* Human-readable name of a status code (static string, never NULL). */
const char* rrs_status_string(int status);

/* Library version string, e.g. "rrs-gfx950 1.0". */
const char* rrs_version(void);

/* Bytes of a code matrix of `rows` rows of length K in the stored layout
 * above (the xq buffer rrs_frontend writes for M = rows tokens). Returns 0
 * for an invalid shape. */
size_t rrs_codes_bytes(int rows, int K);

/* Bytes of the opaque prepared-weight buffer for a [K, N] weight: the packed
 * codes of the N output channels (rrs_codes_bytes(N, K) bytes, stored
 * layout) followed (256-byte aligned) by dw fp32 [N]. Returns 0 for an
 * invalid shape. */
size_t rrs_weight_bytes(int K, int N);

/* Bytes of the workspace that rrs_linear needs for M tokens: a
 * synchronisation block (rrs_sync_bytes(K, G): control words, a reserved
 * area, and a row of K/G 64-bit group-maximum words, tagged with the call
 * count, for each of up to 512 workgroups), then xq (rrs_codes_bytes(M, K)
 * bytes, stored layout), dx [M] and
 * S [K/G], each 256-byte aligned; for K = m 2^k (Kronecker rotation) also a
 * row area of M x K fp32 (the rotated, reordered rows, kept between the
 * front end's stats and quantise passes so that each row is rotated once).
 * rrs_frontend needs only the synchronisation block. Returns 0 for an
 * invalid shape. */
size_t rrs_workspace_bytes(int M, int K, int G);
size_t rrs_sync_bytes(int K, int G);

/* Initialise a workspace: zeroes all `ws_bytes` bytes (the synchronisation
 * block at its start among them) with a fill kernel on `s` (no hipMemset,
 * so it is safe under stream capture). Call once for a fresh workspace
 * before its first use; every later call leaves the block ready for the
 * next one (the one-launch front end counts calls in it instead of
 * clearing it). Two calls that share one workspace must not overlap in
 * time. */
int rrs_workspace_init(void* ws, size_t ws_bytes, hipStream_t s);

/* Calibration reorder (RRS rebuttal page, "Novelty": reorder collects outlier
 * and normal channels). Rotates the T calibration rows X_cal fp16 [T, K],
 * takes each channel's |max| over them and writes perm int32 [K] = channels
 * sorted by that max, largest first, ties by lower channel index.
 * `ws` needs rrs_calibrate_workspace_bytes(K) bytes; it need not be zeroed. */
size_t rrs_calibrate_workspace_bytes(int K);
int rrs_calibrate_perm(const void* X_cal_fp16, int T, int K, int32_t* perm,
                       void* ws, size_t ws_bytes, hipStream_t s);
/* Same with the signed rotation X_cal D H_K. */
int rrs_calibrate_perm_signed(const void* X_cal_fp16, int T, int K,
                              const uint32_t* dsign, int32_t* perm, void* ws,
                              size_t ws_bytes, hipStream_t s);
/* Either of the above (dsign NULL or not) or, with flags =
 * RRS_FLAG_NO_ROTATE, the order of the raw channels' maxima (calibration for
 * Runtime Smooth alone; dsign must be NULL). No other flag is accepted. */
int rrs_calibrate_perm_ex(const void* X_cal_fp16, int T, int K,
                          const uint32_t* dsign, int flags, int32_t* perm,
                          void* ws, size_t ws_bytes, hipStream_t s);

/* Offline weight preparation (output-preserving transform of the AGC-OR page,
 * Sec. 3.1; reorder answer of the RRS rebuttal page; per-output-channel
 * symmetric 4-bit weights, AGC-OR Sec. 5): Wz = H_K W, rows reordered by
 * perm, each output channel quantised with dw[n] = max|col|/7, codes
 * rne(7 Wp/max|col|). Writes the opaque buffer `wq` (rrs_weight_bytes(K, N)
 * bytes). Independent of G: one buffer serves every group size. */
int rrs_prepare_weights(const void* W_fp16, int K, int N, const int32_t* perm,
                        void* wq, hipStream_t s);
/* Same with Wz = H_K D W (the weight side of the signed rotation). */
int rrs_prepare_weights_signed(const void* W_fp16, int K, int N,
                               const int32_t* perm, const uint32_t* dsign,
                               void* wq, hipStream_t s);
/* Either of the above (dsign NULL or not) or, with flags =
 * RRS_FLAG_NO_ROTATE, the weight side of Runtime Smooth alone: Wz = W (no
 * rotation; dsign must be NULL), reordered and quantised the same way. No
 * other flag is accepted (RRS_EINVAL). */
int rrs_prepare_weights_ex(const void* W_fp16, int K, int N,
                           const int32_t* perm, const uint32_t* dsign, int flags,
                           void* wq, hipStream_t s);

/* The RRS A4W4 linear layer: Y fp32 [M, N] = RRS(X) against prepared weights.
 * `ws` holds rrs_workspace_bytes(M, K, G) bytes, initialised once with
 * rrs_workspace_init. Y is fully overwritten. Runs the front end (rotation,
 * reorder, runtime group smoothing, per-token quantise and pack) and the
 * grouped integer GEMM on `s`. The front end's launch may also read wq's
 * codes once ahead of the GEMM (most of them with few tokens, on compute
 * units its rows leave idle; all of them, up to 8 MiB, in its one-launch
 * form before the tiled GEMM) so that the GEMM finds them in the memory-side
 * cache; it writes nothing there, and Y is the same bits as rrs_frontend
 * followed by rrs_gemm. */
int rrs_linear(const void* X_fp16, int M, int K, int N, int G,
               const int32_t* perm, const void* wq, float* Y, void* ws,
               size_t ws_bytes, hipStream_t s);
/* Same with the signed rotation X D H_K (wq from rrs_prepare_weights_signed
 * with the same mask). */
int rrs_linear_signed(const void* X_fp16, int M, int K, int N, int G,
                      const int32_t* perm, const uint32_t* dsign, const void* wq,
                      float* Y, void* ws, size_t ws_bytes, hipStream_t s);

/* The layer with the component switches of the RRS rebuttal page
 * ("Incomplete ablation study": online smoothing, reordering and rotation
 * as separable parts). `flags` as for rrs_frontend:
 *   0                  the full method (same as rrs_linear / _signed);
 *   RRS_FLAG_NO_ROTATE Runtime Smooth alone: no rotation on either side,
 *                      so wq must come from rrs_prepare_weights_ex with
 *                      RRS_FLAG_NO_ROTATE (and perm from calibration on
 *                      the raw channels); Y = dx dw sum_g S_g P_g, with
 *                      no 1/K (no Hadamard pair to undo);
 *   RRS_FLAG_NO_SMOOTH the rotation alone (S = 1): per-token 4-bit
 *                      activations of the rotated rows against the same
 *                      rotated weights, the per-channel A4W4 baseline;
 *   RRS_FLAG_TWO_PASS, RRS_FLAG_TEST_GIVE_UP as for rrs_frontend.
 * dsign: the signed rotation's mask, or NULL (rejected with
 * RRS_FLAG_NO_ROTATE). Mixing weights prepared for one form with another
 * form's call is outside the contract (the buffer does not record it). */
int rrs_linear_ex(const void* X_fp16, int M, int K, int N, int G,
                  const int32_t* perm, const uint32_t* dsign, int flags,
                  const void* wq, float* Y, void* ws, size_t ws_bytes,
                  hipStream_t s);

/* Front end alone (same kernels as rrs_linear): writes the codes xq
 * (rrs_codes_bytes(M, K) bytes, stored layout),
 * dx fp32 [M] and S fp32 [K/G] (zero groups reported as 1). `ws` holds at
 * least rrs_sync_bytes(K, G) bytes, initialised once with
 * rrs_workspace_init. `flags` selects the ablations of the RRS rebuttal page
 * ("Incomplete ablation study"): RRS_FLAG_NO_ROTATE skips the rotation
 * (Runtime Smooth alone), RRS_FLAG_NO_SMOOTH forces S = 1 (rotation alone);
 * 0 is the full method. RRS_FLAG_TWO_PASS changes no result: it makes the
 * smoothed front end use three launches (each workgroup's group maxima,
 * their reduction to S, then quantise; X is read twice), the form
 * rrs_linear falls back to when the one-launch form does not fit on the
 * device at once. That form keeps the per-workgroup maxima in xq, which its
 * last launch then overwrites with the codes.
 *
 * For K = m 2^k with smoothing, up to 256 rows take a one-launch form as
 * well (one workgroup per row, the same grid-wide wait). With more rows, or
 * RRS_FLAG_TWO_PASS, and the rotation on, a `ws` of at least
 * rrs_workspace_bytes(M, K, G) bytes is taken as an rrs_linear workspace:
 * its row area keeps the rotated rows between the stats and quantise passes
 * (as in rrs_linear) unless X, perm, dsign, xq, dx or S lies in that area;
 * with a smaller `ws` the quantise pass rotates every row again. The results
 * are the same bits in every form.
 *
 * The one-launch form keeps every rotated row on chip while the workgroups
 * combine their group maxima, so all its workgroups must be resident
 * together; rrs_linear and rrs_frontend check that against the device's
 * occupancy before choosing it. Its wait is bounded: if the workgroups never
 * all arrive (for example when another such call on another stream holds
 * part of the device), the kernel still ends, with wrong codes, and sets
 * word 2 of the workspace (the error word) to nonzero; the word stays set
 * until rrs_workspace_init. A workgroup that gives up also writes NaN into
 * the token scales dx of its rows (and into S if it is the workgroup that
 * writes S), so a given-up wait never looks like a result; rrs_linear
 * additionally writes NaN into all of Y while the error word is set, and a
 * one-launch front end that finds the error word set gives up at once (no
 * wait), so every later call on that workspace fails the same visible way
 * until it is initialised again.
 * Because of the co-residency requirement, run one-launch calls that share
 * the device on one stream (calls on two streams can starve each other
 * until the spin limit, after which both fail visibly as above).
 *
 * RRS_FLAG_TEST_GIVE_UP exists for tests of that failure path: the
 * one-launch wait gives up at once in every workgroup (error word set,
 * outputs marked), and every kernel still ends normally. It changes
 * nothing in the three-launch form or without smoothing. */
#define RRS_FLAG_NO_ROTATE 1
#define RRS_FLAG_NO_SMOOTH 2
#define RRS_FLAG_TWO_PASS 4
#define RRS_FLAG_TEST_GIVE_UP 8
int rrs_frontend(const void* X_fp16, int M, int K, int G, const int32_t* perm,
                 uint8_t* xq, float* dx, float* S, void* ws, size_t ws_bytes,
                 int flags, hipStream_t s);
/* Same with the signed rotation X D H_K. The signs belong to the rotation:
 * RRS_FLAG_NO_ROTATE together with a sign mask is rejected (RRS_EINVAL). */
int rrs_frontend_signed(const void* X_fp16, int M, int K, int G,
                        const int32_t* perm, const uint32_t* dsign, uint8_t* xq,
                        float* dx, float* S, void* ws, size_t ws_bytes,
                        int flags, hipStream_t s);

/* Number of launches (1 or 3) the front end of rrs_linear / rrs_frontend
 * uses for M tokens of length K with these flags on the current device:
 * 1 when the one-launch form fits on the device at once (or without
 * smoothing; for K = m 2^k up to 256 rows, one workgroup each), 3
 * otherwise. A host-side query; RRS_EINVAL for bad arguments,
 * RRS_EHIP if the device cannot be queried. */
int rrs_frontend_passes(int M, int K, int flags);

/* Grouped integer GEMM alone (same kernels as rrs_linear): Y = (1/K) dx dw
 * sum_g S_g P_g with P_g the int32 group partials of the 4-bit codes; each
 * group's exact partial is multiplied by its smoothing scale S_g before the
 * fp32 accumulation (RRS summary page, "Approach": the scales are not
 * migrated into the weights; RRS rebuttal page, "Novelty": group-wise
 * scales keep the GEMM's tiled scheme). xq (stored layout) and dx fp32 [M]
 * as rrs_frontend writes them, S fp32 [K/G], wq a prepared weight buffer,
 * Y fp32 [M, N] (fully overwritten). The tiled kernel writes the tiles
 * that lie inside Y with streaming (non-temporal) stores, so Y is not left
 * in the caches for a consumer that follows; the few-token kernel loads
 * the weight codes the same way when one 64-token slice streams more than
 * 16 MiB of them. */
int rrs_gemm(const uint8_t* xq, const float* dx, const float* S, int M, int K,
             int N, int G, const void* wq, float* Y, hipStream_t s);

/* Which GEMM kernel rrs_gemm and rrs_linear run for M tokens of length K,
 * N output channels and group size G: RRS_GEMM_TILED (256 x 128 output
 * tiles, every shape) or RRS_GEMM_FEW_TOKENS (one workgroup per 32 output
 * channels and 64 tokens, streaming the weights once per 64 tokens; needs
 * K to split into whole 256-code rounds over 8 waves (K a multiple of
 * 2048) or over 7, 6, 5 or 4 waves, with each wave's run of K and G
 * nested (one a multiple of the other); it serves every M <= 64 and, up to
 * M = 512, the shapes where it needs fewer rounds of workgroups than the
 * tiled kernel, weighted by their measured cost per round). Both apply
 * the same arithmetic (group partials exact, rescaled in fp32). A host-side
 * query; RRS_EINVAL for bad arguments. */
#define RRS_GEMM_TILED 1
#define RRS_GEMM_FEW_TOKENS 2
int rrs_gemm_form(int M, int K, int N, int G);

/* The int32 group partials P[t-m0][n-n0][g] = sum_{j in group g} q[t,j]
 * qw[n,j] for m0 <= t < m1, n0 <= n < n1 (the integer contraction of step 4
 * before its group scales; RRS rebuttal page, "Novelty"), for exactness
 * checks. They come from the same kernel instantiation that rrs_gemm runs
 * for (M, K, N, G) (rrs_gemm_form tells which), with its K split across
 * waves and its rescale points: where that kernel multiplies the
 * accumulator by S_{g-1}/S_g this one multiplies it by 0, and each group's
 * integer sum (or each wave's integer piece of it) is written (added) into
 * P. P is int32 [m1-m0][n1-n0][K/G] (device); xq and wq as for rrs_gemm.
 * The few-token kernel clears the window of P on `s` before adding. */
int rrs_gemm_partials(const uint8_t* xq, int M, int K, int N, int G,
                      const void* wq, int m0, int m1, int n0, int n1,
                      int32_t* P, hipStream_t s);

/* For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): rrs_linear without the
 * caller's workspace. The workspace (synchronisation block, xq, dx, S) is a
 * device array of RRS_NOALLOC_SCRATCH_BYTES inside the library, one per GPU
 * the library runs on, held until the process ends; the call allocates
 * nothing. A call needs rrs_workspace_bytes(M, K, G) bytes of it, less the
 * Kronecker row area (for K = m 2^k the three-launch front end rotates
 * every row twice instead); a larger request returns RRS_ETOOBIG and
 * launches nothing (at K = 4096 every G fits up to M = 11974 tokens, at
 * K = 8192 and G = 128 up to M = 6057). X, perm, wq
 * and Y as for rrs_linear (wq from rrs_prepare_weights).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (it starts zeroed, and the one-launch front end's call count
 * makes clearing between calls unnecessary): calls that overlap in time on
 * one GPU (several streams, or several host threads) race and must not be
 * made. If a one-launch wait ever gives up in it (possible only when other
 * work holds part of the device), every later call on that GPU returns NaN
 * in Y until the process ends. */
#define RRS_NOALLOC_SCRATCH_BYTES ((size_t)24 << 20)
int rrs_linear_noalloc(const void* X_fp16, int M, int K, int N, int G,
                       const int32_t* perm, const void* wq, float* Y,
                       hipStream_t s);

#ifdef __cplusplus
}
#endif

#endif /* RRS_H_ */
