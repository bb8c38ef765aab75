/*
 * tern.h -- C ABI of the MI355X (gfx950) ternary-weight linear layer.
 *
 * The operation (sources cited by page title and section):
 *   y[t][n] = sum_g s[n][g] * sum_{k in group g} w[n][k] * x[t][k]
 * with ternary weights w in {-1, 0, +1} and one fp16 scale s per group of G
 * consecutive weights along the input dimension K ("NInfer sm_89 fork"
 * article, section 9 item 2, which uses G = 128; G = 64 is also accepted),
 * applied to T activation rows x (bf16). The layer picks one of four
 * "rungs" by T ("NINFER ternary perf-tuning" notes, section 2, rung map):
 *   gemv           T = 1 (decode)
 *   small_t        T = 2..8 (draft-verify batches)
 *   small_t_tiled  T = 9..16
 *   s8             T >= 17: activations quantised per token to int8 and the
 *                  product run as an integer contraction (article, sections
 *                  7 and 9 item 2); the only rung that changes numerics
 *                  (notes, section 4).
 *
 * Conventions for every entry point:
 *  - Plain pointers and sizes. "host" pointers are CPU memory; "device"
 *    pointers are HIP device memory on the current device. The caller owns
 *    every buffer; the library allocates no device memory and keeps no
 *    device state.
 *  - Matrices are row-major: x [T][K] bf16 bit patterns (uint16), y [T][N]
 *    float32, w [N][K] int8, scales [N][K/G] fp16 bit patterns (uint16).
 *  - stream is a hipStream_t (NULL = the default stream). Device work is
 *    enqueued asynchronously and the call returns without synchronising;
 *    a kernel fault surfaces at the caller's next synchronisation.
 *  - Every argument is validated on the host before any HIP call. On error
 *    nothing is enqueued, a tern_status other than TERN_OK is returned and
 *    tern_last_error() describes it (thread-local). There is no silent
 *    fallback: a forced rung either runs or returns an error.
 *  - Environment knobs (read once, at the first call that needs them,
 *    validated and then frozen for the life of the process; an invalid value
 *    makes every later tern_linear call fail with TERN_ERR_CONFIG):
 *      TERN_RUNG=auto|gemv|small_t|small_t_tiled|s8   rung for TERN_RUNG_AUTO calls
 *      TERN_S8=0|1                 0 sends T >= TERN_S8_MIN_T to small_t_tiled
 *      TERN_S8_MIN_T=<int>=1..>    first T of the s8 rung (default 17)
 *      TERN_SMALL_T_MAX=<int>      last T of small_t (default 8, at most 16)
 *      TERN_SMALL_T_TILED_MAX=<int> last T of small_t_tiled before s8 (default 16);
 *                                  the same threshold as TERN_S8_MIN_T - 1: set
 *                                  either, or both consistently (else
 *                                  TERN_ERR_CONFIG); at least TERN_SMALL_T_MAX
 *      TERN_DEBUG=0|1, TERN_DEBUG_MIN_T=<int>, TERN_DEBUG_BUDGET=<int>
 *                                  print "rung=<name> T= N= K= G=" lines to
 *                                  stderr for calls with T >= MIN_T, at most
 *                                  BUDGET lines (default 1000)
 *    The rung map, the env-switchable thresholds and the probe follow the
 *    perf-tuning notes, section 2 (every branch must report itself) and
 *    section 7 (decode choices frozen per process).
 */
#ifndef TERN_H
#define TERN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Tag of packed weight layout v1 (stored in tern_weights.layout). */
#define TERN_LAYOUT_V1 0x54524e31u /* "TRN1" */
/* Tag of the base-3 layout t5 (five weights per byte; see below). */
#define TERN_LAYOUT_T5 0x54524e35u /* "TRN5" */

typedef enum {
  TERN_RUNG_AUTO = 0,
  TERN_RUNG_GEMV = 1,
  TERN_RUNG_SMALL_T = 2,
  TERN_RUNG_SMALL_T_TILED = 3,
  TERN_RUNG_S8 = 4,
  TERN_RUNG_COUNT = 5
} tern_rung;

typedef enum {
  TERN_OK = 0,
  TERN_ERR_NULL = 1,      /* a required pointer is NULL */
  TERN_ERR_SHAPE = 2,     /* T < 1 or T > 2^19, N % 16, K % 256, K % G, G not 64/128,
                             K > 2^20 or N > 2^24 (the kernels' 32-bit offsets) */
  TERN_ERR_ALIGN = 3,     /* a device pointer is not 16-byte aligned */
  TERN_ERR_VALUE = 4,     /* a weight outside {-1,0,+1}, a code 10 in packed data */
  TERN_ERR_RUNG = 5,      /* unknown rung, or a forced rung that cannot take this T */
  TERN_ERR_WORKSPACE = 6, /* workspace missing or smaller than tern_workspace_bytes() */
  TERN_ERR_CONFIG = 7,    /* invalid TERN_* environment value */
  TERN_ERR_HIP = 8,       /* a HIP runtime call failed (launch error) */
  TERN_ERR_LAYOUT = 9     /* tern_weights.layout is neither TERN_LAYOUT_V1 nor TERN_LAYOUT_T5,
                             or a t5 matrix on a rung other than gemv */
} tern_status;

/*
 * Packed weight layout v1 (this library's own format; the pages pack base-3,
 * five weights per byte, and pre-lay weights out for their kernels at load
 * time -- "pwwt" engine overview, section 3, weight loader).
 *
 *  - N % 16 == 0, K % 256 == 0, G in {64, 128}.
 *  - 2-bit code per weight: 00 -> 0, 01 -> +1, 11 -> -1; 10 is never written
 *    and is rejected by tern_unpack.
 *  - Strip s = rows [16s, 16s+16); k-tile kt = columns [256kt, 256kt+256).
 *    Tile (s, kt) is 1024 bytes at byte offset (s*KT + kt)*1024, KT = K/256,
 *    so one strip's k-tiles are contiguous (KT KiB per strip).
 *  - Inside a tile, lane L in [0, 64) owns bytes [16L, 16L+16), read as four
 *    little-endian 32-bit words P[0..3].
 *  - Weight (row 16s + r, column 256kt + kk) with kk = 32m + 8g + 2d + h,
 *    m in [0,8), g in [0,4), d in [0,4), h in {0,1}: lane L = 16g + r, word
 *    P[m >> 1], j = 4*(m & 1) + d, and the code occupies bits [b+1 : b] with
 *    b = (h ? 30 : 14) - 2j.
 *    (Shifting P left by 2j and masking 0xC000C000 leaves the two codes of a
 *    bf16 pair at bits 15:14 and 31:30: 0x4000 = +2.0, 0xC000 = -2.0, 0 = 0.)
 *  - Scales are re-laid as [s][kt][r][gi], gi in [0, 256/G): element
 *    ((s*KT + kt)*16 + r)*(256/G) + gi holds scale[16s + r][kt*(256/G) + gi].
 *  - Sizes: N*K/4 bytes of codes, N*(K/G)*2 bytes of scales.
 */
/*
 * Base-3 layout t5: five weights per byte, the "t5" ternary format of the
 * "NInfer sm_89 fork" article, section 9 item 2, laid out here for the
 * integer matrix core. 13 bytes per 64 weights (1.625 bits per weight, 19 %
 * fewer code bytes than v1). Only the gemv rung (T = 1) reads it.
 *
 *  - N % 16 == 0, K % 1024 == 0, G in {64, 128}; a weight w is the trit
 *    t = w + 1 in {0, 1, 2}.
 *  - Strip s = rows [16s, 16s+16); k-quad Q = columns [1024Q, 1024Q+1024),
 *    four k-tiles j = 0..3. Block (s, Q) is 3328 bytes at byte offset
 *    (s*KQ + Q)*3328, KQ = K/1024.
 *  - In a block, k-tile j's main part is bytes [768j, 768j+768): lane
 *    L in [0, 64) owns bytes [768j + 12L, +12), little-endian words W0..W2.
 *    Bytes [3072, 3328) are tails: byte 3072 + 4L + j is lane L's tail byte
 *    of k-tile j.
 *  - Weight (row 16s + r, column 1024Q + 256j + kk), kk = 64q + u: with
 *    hi = (u >= 32), u' = u - 32 hi, g = u' / 8, p = u' % 8, i = p / 2 and
 *    e = hi ? (p odd ? 2 : 0) : (p odd ? 3 : 1), it is byte e of register
 *    R = 4q + i of lane L = 16g + r (the order of TERN_Q_OPERAND_ORDER).
 *  - R < 15: byte e of word W[R / 5] holds five trits t_0..t_4 of
 *    registers 5(R/5) .. 5(R/5)+4 (digit d = R % 5, t_0 most significant)
 *    as v = sum_d t_d 3^(4-d), stored as the byte ceil(256 v / 243).
 *  - R == 15: bits [2e+1 : 2e] of the tail byte hold the trit.
 *  - Scales as in layout v1. Sizes: N*(K/1024)*208 code bytes.
 */

typedef struct {
  const void* codes;      /* device, N*K/4 bytes (v1) or N*(K/1024)*208 (t5), 16-byte aligned */
  const uint16_t* scales; /* device, N*(K/G) fp16 in the re-laid order, 16-byte aligned */
  int32_t n;              /* output features N */
  int32_t k;              /* input features K */
  int32_t group;          /* G: 64 or 128 */
  uint32_t layout;        /* TERN_LAYOUT_V1 or TERN_LAYOUT_T5 */
} tern_weights;

/* Bytes of packed codes for an N x K matrix (N*K/4), 0 if the shape is invalid. */
size_t tern_packed_code_bytes(int n, int k);
/* Number of fp16 scales (N*(K/G)), 0 if the shape is invalid. */
size_t tern_scale_count(int n, int k, int group);

/*
 * Offline relayout (host, synchronous): int8 weights w [N][K] (host) and fp16
 * scales [N][K/G] (host, bit patterns) -> packed codes (host, N*K/4 bytes)
 * and re-laid scales (host, N*(K/G) uint16). Copy both to the device and
 * describe them with a tern_weights. Errors: TERN_ERR_NULL, TERN_ERR_SHAPE,
 * TERN_ERR_VALUE (a weight outside {-1,0,+1}; outputs are then undefined).
 */
tern_status tern_pack(const int8_t* w, const uint16_t* scales_f16, int n, int k, int group,
                      void* codes_out, uint16_t* scales_out);

/* Inverse of tern_pack (host, synchronous). scales_packed and scales_out may be
 * NULL to skip the scales. TERN_ERR_VALUE if a code 10 is found. */
tern_status tern_unpack(const void* codes, const uint16_t* scales_packed, int n, int k,
                        int group, int8_t* w_out, uint16_t* scales_out);

/* Bytes of t5 codes for an N x K matrix (N*(K/1024)*208), 0 if the shape is
 * invalid for t5 (N % 16, K % 1024). */
size_t tern_packed_code_bytes_t5(int n, int k);
/* tern_pack into the base-3 layout t5 (host, synchronous): the same inputs,
 * tern_packed_code_bytes_t5(n, k) bytes of codes, scales re-laid as for v1.
 * Errors: TERN_ERR_NULL, TERN_ERR_SHAPE (K % 1024 too), TERN_ERR_VALUE. */
tern_status tern_pack_t5(const int8_t* w, const uint16_t* scales_f16, int n, int k, int group,
                         void* codes_out, uint16_t* scales_out);
/* Inverse of tern_pack_t5 (host, synchronous); TERN_ERR_VALUE for a byte that
 * tern_pack_t5 never writes (not ceil(256 v / 243) for v <= 242) or a tail
 * trit of 3. scales_packed and scales_out may both be NULL. */
tern_status tern_unpack_t5(const void* codes, const uint16_t* scales_packed, int n, int k,
                           int group, int8_t* w_out, uint16_t* scales_out);

/* Layouts of int8 activations q [T][K]. */
typedef enum {
  TERN_Q_ROW_MAJOR = 0,     /* q[t][k] at byte t*K + k */
  TERN_Q_OPERAND_ORDER = 1  /* K % 64 == 0; inside row t, the byte at 64b + 16g + 4i + e holds
                               k = 64b + 8g + m(i, e), m(i, .) = {32+2i, 2i, 33+2i, 2i+1}: the
                               order in which the s8 contraction consumes a 64-wide k-block */
} tern_q_layout;

/*
 * Per-token symmetric int8 activation quantisation (device, async), the first
 * step of the s8 rung ("NInfer sm_89 fork" article, section 7 and section 9
 * item 2):
 *   a_t = max_k |x[t][k]|;  scale_t = fl32(a_t / 127) (IEEE division);
 *   q[t][k] = clamp(round-half-even(fl32(x[t][k] / scale_t)), -127, 127);
 *   a_t == 0 gives scale_t = 0 and q[t][:] = 0.
 * x: device bf16 [T][K]; q: device int8 [T][K] in `layout`; act_scale: device
 * float [T]. K % 8 == 0 (K % 64 == 0 for TERN_Q_OPERAND_ORDER); x and q
 * 16-byte aligned.
 */
tern_status tern_quant_act_s8(const void* x_bf16, int T, int k, int8_t* q, float* act_scale,
                              tern_q_layout layout, void* stream);

/*
 * Rotated per-token int8 activation quantisation (device, async): the
 * Hadamard rotation that the pages fold into the activation quantisation
 * ("NInfer sm_89 fork" article, section 9 item 2), on 1024-wide blocks
 * ("NINFER ternary perf-tuning" notes, section 6, constants table), in the
 * same kernel as the quantisation:
 *   xr[t][1024b + i] = (1/32) sum_j H[i][j] x[t][1024b + j],
 *     H[i][j] = (-1)^popcount(i & j) (Sylvester, order 1024), computed in
 *     fp32 as the fast Walsh-Hadamard transform with strides 1, 2, ..., 512
 *     in that order (each pair (u, v) -> (u + v, u - v), one rounding each),
 *     then one multiply by 1/32;
 *   then tern_quant_act_s8's rule on xr: a_t = max_k |xr[t][k]|,
 *   scale_t = fl32(a_t / 127), q = clamp(round-half-even(fl32(xr / scale_t)),
 *   -127, 127); a_t == 0 gives scale_t = 0 and zero codes.
 * The result feeds tern_linear_s8_q with weights trained in the rotated basis.
 * x: device bf16 [T][K]; q: device int8 [T][K] in `layout`; act_scale: device
 * float [T]. K a multiple of 1024 in [1024, 32768]; x and q 16-byte aligned.
 * The caller keeps |x| small enough that the block sums stay finite.
 * Errors: TERN_ERR_NULL, TERN_ERR_SHAPE, TERN_ERR_VALUE (layout),
 * TERN_ERR_ALIGN, all before any launch; TERN_ERR_HIP if the launch fails.
 */
tern_status tern_quant_act_s8_rot(const void* x_bf16, int T, int k, int8_t* q, float* act_scale,
                                  tern_q_layout layout, void* stream);

/*
 * Device workspace tern_linear needs for this call (bytes, 0 if none). The s8
 * rung keeps the int8 activations and their scales there, and on short
 * prefills of narrow layers also fp32 partial totals when it splits K across
 * workgroups (a second kernel adds them in a fixed order); small_t and
 * small_t_tiled (up to 16 tokens) keep fp32 partial sums there when they
 * split K across workgroups (narrow layers with a long K; then a second
 * kernel adds the parts in a fixed order). (On wide layers at T <= 4 the
 * int8 limbs of the activations are made inside the contraction kernel and
 * need none; forced with TERN_TUNE_SMALLT=limb2, or at T = 5..8 with
 * TERN_TUNE_SMALLT=limb, a prep kernel keeps them and their per-k-tile
 * exponents here.) Whenever this is not 0 it includes a header of 4096
 * bytes at the start of the workspace, which only the narrow-layer kernel
 * (TERN_KERNEL_SMALLT_NARROW) uses: arrival counters that must be zero before
 * the workspace's first use (one hipMemset) and that every call leaves zero,
 * also when calls of other rungs share the workspace. The rest needs no
 * initialisation and is not preserved. Every scratch buffer of every rung is
 * counted here; a call given less fails with
 * TERN_ERR_WORKSPACE ("NINFER ternary perf-tuning" notes, section 5 item 8:
 * the workspace capacity declaration must cover every scratch).
 * rung may be TERN_RUNG_AUTO (resolved the way tern_linear resolves it).
 * Returns (size_t)-1 for an invalid shape, rung or configuration.
 */
size_t tern_workspace_bytes(int T, int n, int k, int group, tern_rung rung);

/*
 * y = ternary_linear(x) (device, async).
 *  x:  device bf16 [T][K], 16-byte aligned
 *  W:  host struct describing device codes and scales (layout v1)
 *  y:  device float [T][N], 16-byte aligned; fully overwritten
 *  rung: TERN_RUNG_AUTO picks by T (after TERN_RUNG); any other value forces
 *        that rung. small_t takes T <= 16 (one 16-token tile); gemv takes
 *        T <= 65535; small_t_tiled and s8 take any T >= 1 (small_t_tiled
 *        above 16 tokens runs the bf16 prefill contraction, the path T >= 17
 *        takes with TERN_S8=0).
 *  ws, ws_bytes: device workspace (16-byte aligned) of at least
 *        tern_workspace_bytes(T, N, K, G, rung) bytes (may be NULL/0 if that is 0)
 * Output numerics: the bf16-activation rungs (gemv, small_t, small_t_tiled)
 * accumulate exact bf16 x {-1,0,+1} products in fp32, except that the gemv
 * kernel and, on wide layers at T <= 4, small_t and small_t_tiled carry each
 * activation as a 22-bit fixed-point number relative to
 * the largest magnitude M of its 256-wide k-tile (exact for values down to
 * 2^-14 M, rounded by at most 2^-22 M below that); s8 computes exact int32
 * group accumulators and y = scale_t * sum_g s[n][g] * acc in fp32, groups in
 * ascending order (when K is split across workgroups: ascending within each
 * part, then the parts' totals added in ascending order).
 */
tern_status tern_linear(const void* x_bf16, int T, const tern_weights* W, float* y,
                        tern_rung rung, void* ws, size_t ws_bytes, void* stream);

/* Bytes of the static device scratch behind tern_linear_noalloc (64 MiB). */
#define TERN_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * tern_linear without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc): the same rungs, kernels and results as
 * tern_linear, with the workspace taken from a static device scratch of
 * TERN_NOALLOC_SCRATCH_BYTES that the library holds on each GPU it runs on
 * until the process ends. The call allocates nothing; it needs no
 * initialisation of the scratch (it is zero when the library is loaded, the
 * counter header of tern_workspace_bytes stays zero after every call, and
 * every kernel writes the rest before it reads it).
 *  - A call whose tern_workspace_bytes() exceeds TERN_NOALLOC_SCRATCH_BYTES
 *    fails with TERN_ERR_WORKSPACE before any HIP call (e.g. the s8 rung
 *    from about 3,800 tokens at K = 17408).
 *  - The first call on each device resolves the scratch's device address
 *    (a HIP symbol lookup, no allocation): make it outside graph capture.
 *  - All calls on one GPU share its scratch, which keeps the last call's
 *    contents: calls that can overlap on one GPU (other streams, other
 *    threads) race on it. Serialise them, or use tern_linear with a
 *    workspace per stream.
 * Arguments and errors as tern_linear (TERN_ERR_HIP also if the symbol
 * lookup fails).
 */
tern_status tern_linear_noalloc(const void* x_bf16, int T, const tern_weights* W, float* y,
                                tern_rung rung, void* stream);

/*
 * A whole decode pass in one launch: a chain of T = 1 projections (the gemv
 * rung's arithmetic and K split, bit-identical results) run by one
 * persistent kernel, one workgroup per CU, whose waves stream the codes of
 * the next projection while they finish the previous one, instead of each
 * launch paying its own ramp and tail ("NINFER ternary perf-tuning" notes,
 * section 6: a decode round is one graph of about 1224 kernels; "NInfer
 * sm_89 fork" article, section 9 item 5: each decode round replayed as one
 * graph).
 *
 * Dependencies: item i with after = j (j < i) reads its x only once items
 * 0..j have all finished (their y and y_bf16 stores visible), e.g. x of item
 * i = y_bf16 of item j; after = -1 reads x at any time. Completion goes
 * through device-scope counters in caller memory, and y, y_bf16 and x move
 * with device-coherent stores and loads; every
 * wait polls at most spin_limit times (each poll sleeps about 0.05 us plus
 * a memory round trip), then sets *error_flag = 1 and the rest of the chain
 * is skipped: the kernel always exits, and the results are then undefined.
 */
typedef struct {
  tern_weights W;   /* layout v1; every item of a chain has the same group size */
  const void* x;    /* device bf16 [K], 16-byte aligned */
  float* y;         /* device fp32 [N], 16-byte aligned; fully overwritten */
  uint16_t* y_bf16; /* device bf16 [N] or NULL: y rounded to nearest even (finite y) */
  int32_t after;    /* -1, or j < the item's index: x is read once items 0..j are done */
} tern_chain_item;

/* Host-side summary of a built chain, filled by tern_chain_build. */
typedef struct {
  int32_t count;      /* items */
  int32_t group;      /* their group size */
  int32_t workgroups; /* workgroups of the launch (one per CU) */
  int32_t lds_bytes;  /* dynamic LDS per workgroup */
  int32_t waits;      /* 1 if some item waits: the launch is then cooperative */
} tern_chain_plan;

/* Device bytes to allocate for the chain table of these items: enough for
 * any device (up to 512 workgroups); 0 if the chain is invalid
 * (tern_last_error says why). */
size_t tern_chain_table_bytes(const tern_chain_item* items, int count);
/* Device bytes of the completion counters of `count` items (count + 1 ints). */
size_t tern_chain_counter_bytes(int count);
/*
 * Validates the chain (host), splits every item's K as the gemv rung does,
 * cuts the chain into stages at the items that wait, gives each of one
 * workgroup per CU of the current device a contiguous run of every stage's
 * work, balanced by bytes, expands it into the list of tasks and
 * synchronisation points each of the workgroup's waves walks, and writes
 * the table (device memory, at least
 * tern_chain_table_bytes(items, count) bytes, 16-byte aligned) with one
 * synchronous host-to-device copy. Build once per set of buffers; the table
 * holds the pointers of items[]. The limbs of two items' activations share
 * the LDS, so the largest K is about 26,000. Errors: TERN_ERR_NULL,
 * TERN_ERR_SHAPE (count < 1, shapes, mixed group sizes, K too large for the
 * LDS), TERN_ERR_VALUE (after out of range), TERN_ERR_LAYOUT,
 * TERN_ERR_ALIGN, TERN_ERR_WORKSPACE (table too small), TERN_ERR_HIP
 * (device query or copy).
 */
tern_status tern_chain_build(const tern_chain_item* items, int count, void* table, size_t table_bytes,
                             tern_chain_plan* plan);
/*
 * Runs a built chain (device, async, one launch; cooperative, so that
 * every workgroup is resident, when some item waits). counters:
 * device, tern_chain_counter_bytes(count), zeroed before the first call and
 * left zeroed by every call (the last workgroup out clears them); calls that
 * share counters must not overlap. error_flag: device int32, set to 1 if a
 * wait gave up or the table does not match the plan (the caller zeroes it).
 * spin_limit >= 1. TERN_ERR_HIP if the launch is refused. A cooperative launch has a fixed cost of its own (about
 * 10-20 us measured per launch): chains pay off for whole passes.
 */
tern_status tern_linear_chain(const tern_chain_plan* plan, const void* table, void* counters,
                              size_t counter_bytes, int32_t* error_flag, int spin_limit, void* stream);

/*
 * The s8 rung's contraction on activations already quantised by
 * tern_quant_act_s8 (device, async): y[t][n] = scale_t * sum_g s[n][g] *
 * acc[t][n][g] in fp32, groups ascending -- the same kernel and numerics as
 * tern_linear(..., TERN_RUNG_S8, ...) after its quantisation step (which uses
 * TERN_Q_OPERAND_ORDER), except that this call never splits K (it takes no
 * workspace). Lets a caller quantise one activation once and apply
 * several projections to it. q: device int8 [T][K] in `layout` (16-byte
 * aligned); act_scale: device float [T]; y: device float [T][N] (16-byte
 * aligned). Counts as an s8 launch in the probe.
 */
tern_status tern_linear_s8_q(const int8_t* q, const float* act_scale, int T,
                             const tern_weights* W, float* y, tern_q_layout layout, void* stream);

/*
 * Debug export of the s8 rung's integer group accumulators (device, async):
 * acc[t][n][g] = sum_{k in group g} q[t][k] * w[n][k], int32 [T][N][K/G].
 * Runs the s8 contraction kernel that tern_linear_s8_q runs for `layout`
 * (TERN_Q_OPERAND_ORDER: the one tern_linear's s8 rung uses) with its
 * epilogue replaced by a store of the accumulators, so the integer path can
 * be checked bit for bit. q: device int8 [T][K] in `layout`, 16-byte aligned.
 */
tern_status tern_debug_s8_acc(const int8_t* q, int T, const tern_weights* W, int32_t* acc_out,
                              tern_q_layout layout, void* stream);

/*
 * Streaming-read ceiling (device, async): one launch that reads `bytes` of
 * device memory at `buf` once, with 128-bit non-temporal loads and no other
 * work, so that its duration is the floor of any single launch that streams
 * as many bytes. The tuning notes on the pages rate the decode kernels
 * against such a self-measured read-only ceiling ("NINFER ternary
 * perf-tuning" notes, section 6, measured constants).
 *   buf: device, 16-byte aligned, `bytes` readable; bytes a positive
 *        multiple of 1024.
 *   depth: loads in flight per wave, 4, 8 or 16; waves_per_cu: 1..32, the
 *        number of waves per CU the bytes are spread over (one contiguous run
 *        per wave). The fastest pair depends on the size; sweep a few.
 *   sink: device, one uint32; written only when the XOR of a lane's loads
 *        equals an arbitrary constant, so normally left untouched.
 * Errors: NULL pointers (TERN_ERR_NULL), bad size (TERN_ERR_SHAPE), bad
 * depth or waves (TERN_ERR_VALUE), misalignment (TERN_ERR_ALIGN); launch
 * failures TERN_ERR_HIP. Counts as no rung in the probe.
 */
tern_status tern_stream_read(const void* buf, size_t bytes, int depth, int waves_per_cu,
                             uint32_t* sink, void* stream);

/* Rung probe: number of kernel launches per rung since the last reset,
 * counted at the launch site of the kernel that actually ran. */
void tern_probe_snapshot(uint64_t out[TERN_RUNG_COUNT]);
/* Resets the rung probe and the kernel probe. */
void tern_probe_reset(void);

/*
 * Kernel probe: every kernel this library launches, one id each. A rung is
 * served by several kernels chosen by layer shape (and by TERN_TUNE_* knobs),
 * so the rung probe alone cannot say which one produced a result; the kernel
 * probe counts every successful launch per kernel, at its launch site
 * ("NINFER ternary perf-tuning" notes, section 2: every reachable branch
 * reports itself).
 */
typedef enum {
  TERN_KERNEL_QUANT_S8 = 0,       /* per-token int8 quantisation, q in operand order (s8 rung) */
  TERN_KERNEL_QUANT_S8_ROW,       /* the same with row-major q (tern_quant_act_s8 only) */
  TERN_KERNEL_QUANT_S8_ROT,       /* Hadamard-rotated quantisation (tern_quant_act_s8_rot) */
  TERN_KERNEL_GEMV_LIMB,          /* gemv: x as int8 limbs on the i8 matrix cores */
  TERN_KERNEL_GEMV_BF16,          /* gemv: bf16-operand kernel with one-token rows (limbs do not fit LDS) */
  TERN_KERNEL_SMALLT_RESIDENT,    /* small_t: limb kernel, every token's limbs resident in LDS */
  TERN_KERNEL_SMALLT_LIMB_FUSED,  /* small_t: limb contraction, limbs made by a loader wave */
  TERN_KERNEL_SMALLT_LIMB_PREP,   /* small_t: separate limb preparation (limbs to the workspace) */
  TERN_KERNEL_SMALLT_LIMB_TILE,   /* small_t: limb contraction on the prepared limbs */
  TERN_KERNEL_SMALLT_WAVE,        /* small_t / small_t_tiled: per-wave bf16 kernel, 16-token tile */
  TERN_KERNEL_SMALLT_TILE,        /* small_t / small_t_tiled: activation tile shared in LDS */
  TERN_KERNEL_SMALLT_TILE_REDUCE, /* adds the K-split partial sums of SMALLT_TILE */
  TERN_KERNEL_B16_PREFILL,        /* small_t_tiled above 16 tokens: bf16 MFMA contraction */
  TERN_KERNEL_S8_MMA,             /* s8 contraction on operand-order q */
  TERN_KERNEL_S8_REDUCE,          /* adds the K-split partial totals of S8_MMA */
  TERN_KERNEL_S8_ROW,             /* s8 contraction on row-major q (tern_linear_s8_q) */
  TERN_KERNEL_S8_ACC_EXPORT,      /* tern_debug_s8_acc */
  TERN_KERNEL_STREAM_READ,        /* tern_stream_read */
  TERN_KERNEL_GEMV_T5,            /* gemv on base-3 (t5) weights: limbs of x on the i8 matrix cores */
  TERN_KERNEL_CHAIN,              /* tern_linear_chain: a chain of T = 1 projections in one launch */
  TERN_KERNEL_SMALLT_NARROW,      /* small_t / small_t_tiled on narrow layers: K split over workgroups, partials added in-launch */
  TERN_KERNEL_COUNT
} tern_kernel;

/* Launches per kernel since the last tern_probe_reset (all threads). */
void tern_kernel_probe_snapshot(uint64_t out[TERN_KERNEL_COUNT]);
/* Bit i set: kernel i was launched by the most recent successful call on this
 * thread of tern_linear, tern_linear_s8_q, tern_debug_s8_acc,
 * tern_quant_act_s8, tern_quant_act_s8_rot or tern_stream_read (0 before
 * any). With TERN_DEBUG=1 the rung line of tern_linear names them too. */
uint64_t tern_last_kernels(void);
/* Host-only dry run of the dispatcher (no HIP call): the kernel-id bit mask
 * (as tern_last_kernels) that tern_linear(T, N, K, G, rung) on weights of
 * `layout` would launch
 * under the frozen configuration, 0 if the shape, rung or configuration is
 * invalid (tern_last_error says why). */
uint64_t tern_plan_kernels(int T, int n, int k, int group, uint32_t layout, tern_rung rung);
/* Name of a kernel id ("gemv_limb", "smallt_tile", ...; "invalid" if out of range). */
const char* tern_kernel_name(tern_kernel kernel);
/* Rung of the most recent successful tern_linear call on any thread
 * (TERN_RUNG_AUTO if none yet). */
tern_rung tern_last_rung(void);
/* The rung tern_linear would run for (T, rung) under the frozen
 * configuration, or minus the tern_status it would fail with (with
 * tern_last_error set). */
int tern_resolve_rung(int T, tern_rung rung);
/* Name of a rung ("gemv", "small_t", "small_t_tiled", "s8", "auto"). */
const char* tern_rung_name(tern_rung rung);
/* Message of the last error on this thread ("" if none). */
const char* tern_last_error(void);
/* ABI version of this library (currently 1). */
int tern_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TERN_H */
