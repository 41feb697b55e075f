// Internal declarations shared by the HIP sources of libsdm (not installed).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sdm {

constexpr int kMaxK = 64;         // largest W or R
constexpr int kMaxSqrtN = 1024;   // largest sqrtN (N <= 2^20 slots)
constexpr int kMaxDepth = 8;      // largest cross-token prefetch depth

// A slot word of a token record: the slot index in the low 20 bits; the
// planner adds a forwarding code above it when an earlier token (at most
// kMaxDepth-1 tokens back, or the same token for a read) wrote the slot.
constexpr int kSlotBits = 20;
constexpr uint32_t kSlotMask = (1u << kSlotBits) - 1u;
constexpr int kFwdWShift = 20;              // position w' in that token's write list
constexpr uint32_t kFwdWMask = 63u;
constexpr int kFwdDShift = 26;              // token distance d = t - t'
constexpr uint32_t kFwdDMask = 7u;
constexpr uint32_t kFwdValid = 1u << 29;

// Per (chain, token) record written by select and consumed by the write/read
// kernels.  A chain is one (sequence b, head h); records of a chain are
// contiguous in t.  Every array has kMaxK entries whatever W and R are: the
// serial kernel's row groups load their references unconditionally (masked
// entries are ignored), and those loads then always stay inside the record.
//   ws[Wp]  write slot words     wa[Wp]  alpha*(1 - beta*k)   wc[Wp]  beta*k
//   rs[Rp]  read slot words      rq[Rp]  q weights            wk[Wp]  k weights
// (wk is read by the backward only.)
struct RecLayout {
    int Wp, Rp;
    __host__ __device__ RecLayout(int, int) : Wp(kMaxK), Rp(kMaxK) {}
    __host__ __device__ int ws() const { return 0; }
    __host__ __device__ int wa() const { return Wp; }
    __host__ __device__ int wc() const { return 2 * Wp; }
    __host__ __device__ int rs() const { return 3 * Wp; }
    __host__ __device__ int rq() const { return 3 * Wp + Rp; }
    __host__ __device__ int wk() const { return 3 * Wp + 2 * Rp; }
    __host__ __device__ int dwords() const { return 4 * Wp + 2 * Rp; }
};

// One write event of an epoch after sorting by slot (time-parallel schedule):
// slot, token within the epoch << 6 | position w, and the coefficients.
struct TPEntry {
    uint32_t slot, tw;
    float a, c;
};

// Element type of the state M.  float32; bfloat16; or 8-bit OCP FP8 E4M3
// codes scaled by a power of two 2^s (a code c holds the value c * 2^s).
enum StateType : int { kStateF32 = 0, kStateBF16 = 1, kStateFP8 = 2 };
struct StateFmt {
    int type = kStateF32;
    int scale_log2 = 0;  // s (E4M3 state only)
};

// Nearest bfloat16 values (ties to even) of two finite floats, packed: a in
// the low 16 bits, b in the high.  gfx950's v_cvt_pk_bf16_f32 does this in
// one instruction; it gives the bits (u + 0x7FFF + ((u >> 16) & 1)) >> 16 of
// the nearest-even rule for every finite float32 u, subnormals included
// (checked over all of them with denormals enabled, as this library builds).
typedef __bf16 sdm_bf16x2 __attribute__((ext_vector_type(2)));
typedef float sdm_f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pack2(float a, float b)
{
    const sdm_f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, sdm_bf16x2));
}

// E4M3 codes (OCP FP8: sign, 4 exponent bits with bias 7, 3 mantissa bits;
// normal values (1 + m/8) 2^(e-7), subnormals m 2^-9; largest magnitude 448,
// no infinities).  The rule: the nearest code, ties to even, magnitudes
// beyond 448 saturated to 448.  gfx950's conversion instructions use this
// format and round to nearest even, subnormals included (checked against a
// bit-level implementation of the rule over every float32 of magnitude <=
// 448), so the saturation is a clamp before them.
__device__ __forceinline__ float e4m3_clamp(float a)
{
    return __builtin_fminf(__builtin_fmaxf(a, -448.0f), 448.0f);
}

// Codes of a and b in bytes 0 and 1 (HIGH = false) or 2 and 3 (HIGH = true)
// of `old`, the other two bytes kept.
template <bool HIGH>
__device__ __forceinline__ uint32_t e4m3_pack2(float a, float b, uint32_t old)
{
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(e4m3_clamp(a), e4m3_clamp(b), (int)old, HIGH);
}

// Codes of the 4 values, column k in byte k.
__device__ __forceinline__ uint32_t e4m3_pack4(float x, float y, float z, float w)
{
    return e4m3_pack2<true>(z, w, e4m3_pack2<false>(x, y, 0u));
}

// Value of byte k (0..3) of a word of E4M3 codes (exact in float32).
template <int K>
__device__ __forceinline__ float e4m3_value(uint32_t w)
{
    return __builtin_amdgcn_cvt_f32_fp8((int)w, K);
}

struct Shape {
    int B;
    int64_t T;
    int H, sqrtN, d_v, W, R;
    int64_t N() const { return (int64_t)sqrtN * sqrtN; }
    int64_t ht() const { return (int64_t)B * T * H; }
};

// ---- launchers (each returns the launch error, if any) ----

// State initialisation M[b] <- M_0 (every sequence b) carried out by the
// selection launch: each item (head-token and list) copies one 1 KB piece of
// M_0, loaded when the item starts and stored B times when it ends, so the
// copy runs under the selection's arithmetic.  Possible when the items cover
// M_0 that way (select_can_init); M is float32, or bfloat16 (rounded to
// nearest, ties to even).
struct SelInit {
    const float *M0;
    void *M;
    bool state_bf16;  // else float32 (the selection does not carry an E4M3 copy)
};
bool select_can_init(const Shape &s);

// Selection.  With hist != nullptr it only counts write slots per head into
// hist[H][N]; else with rec == nullptr it writes the API layout (Iw, kw, Ir,
// qw, [B][T][H][K]); otherwise it writes token records (needs alpha, beta).
hipError_t launch_select(const Shape &s, const void *kp, const void *qp, bool bf16,
                         int32_t *Iw, float *kw, int32_t *Ir, float *qw,
                         uint32_t *rec, const float *alpha, const float *beta,
                         hipStream_t st, uint32_t *hist = nullptr, int64_t t0 = 0,
                         int64_t tn = -1,  // tokens [t0, t0 + tn) of every sequence
                         const SelInit *init = nullptr);

// M[b] <- M0 for every sequence b, in the state's element type.
hipError_t launch_init(const Shape &s, const float *M0, void *M, StateFmt fmt, hipStream_t st);

// Adds forwarding codes (distance < depth) to the slot words of all records.
hipError_t launch_plan(const Shape &s, uint32_t *rec, int depth, hipStream_t st);

// Token-serial write/read over the records (float4 path): needs d_v % 4 == 0
// and one chain's state within 2^31 bytes.
bool rw_serial_supported(const Shape &s);
hipError_t launch_rw_serial(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st);
int rw_serial_depth(const Shape &s);  // prefetch depth of the serial kernel that runs s

// Token-serial write/read, one column per lane, no prefetch (any d_v).
hipError_t launch_rw_simple(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st);

// Time-parallel schedule (epochs of tokens, slot-sorted write events).
bool tp_supported(const Shape &s);
// Tokens per epoch and workspace beyond the token records; `stored`: a
// bfloat16 or E4M3 state (its epochs may be shorter, see tp_epoch_len).
int tp_epoch_len(const Shape &s, bool stored = false);
size_t tp_workspace_bytes(const Shape &s, bool stored = false);
// Epochs [ep0, ep1) (ep1 < 0: through the last epoch).  With `stored` (a
// bfloat16 or E4M3 state) the read plan is the one of stored-value reads
// (rows rounded after every write): weights q and each read's in-epoch
// writes.
hipError_t launch_tp_prepare(const Shape &s, const uint32_t *rec, void *ws, hipStream_t st,
                             int ep0 = 0, int ep1 = -1, bool link = true, bool stored = false);
hipError_t launch_tp_apply(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                           bool bf16, float *y, void *M, StateFmt fmt, hipStream_t st,
                           int ep0 = 0, int ep1 = -1);

// One-token step (T == 1): the token's writes, then its reads, in one kernel
// (d_v % 4 == 0 and one chain's state within 2^31 bytes).
bool decode_supported(const Shape &s);
hipError_t launch_rw_decode(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, void *M, StateFmt fmt, hipStream_t st);
// The whole one-token step in one launch: each workgroup selects its
// chain's write and read slots itself (no token records) and then writes and
// reads a range of row slices.  Results bit-identical to launch_select +
// launch_rw_decode.  For decode_supported shapes with sqrtN <= 512.
bool decode_fused_supported(const Shape &s);
hipError_t launch_decode_fused(const Shape &s, const void *kp, const void *qp, const void *v,
                               bool bf16, const float *alpha, const float *beta, float *y,
                               void *M, StateFmt fmt, hipStream_t st);
// Compute units of the current device (queried once per device).
int compute_units();
// Candidate columns of stage 2 for lists of K slots (kTabMax entries, pairs
// a << 8 | b) and the number of pairs with both ranks >= 2.
const uint16_t *hook_columns(int K, int *rest);

// Backward (float32 state): a forward write pass over epochs [ep0, ep1) that
// records each written slot's epoch-start row in the tape ([chain][tapeT][W]
// [d_v], token t at entry t - tape_t0), or, with tape == nullptr, only
// advances the state; the write and read events of every epoch sorted
// together by slot; the reverse pass.
hipError_t launch_tp_forward_tape(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                                  bool bf16, float *M, float *tape, int64_t tapeT,
                                  int64_t tape_t0, int ep0, int ep1, hipStream_t st);
hipError_t launch_tp_sort_merged(const Shape &s, const uint32_t *rec, void *ws, TPEntry *out,
                                 uint64_t *tmpA, uint64_t *tmpB, hipStream_t st);
// The backward runs the sequence in `chunks` chunks of whole epochs (1 ..
// number of epochs; 0: the count that needs the least memory): the tape
// holds one chunk, and the state at every chunk start is kept.
int tp_backward_epochs(const Shape &s);
int tp_backward_min_chunks(const Shape &s);
size_t tp_backward_workspace_bytes(const Shape &s, int chunks);  // beyond the forward's workspace
hipError_t launch_tp_backward(const Shape &s, int chunks, const uint32_t *rec, void *fwd_ws,
                              void *bwd_ws, const void *v, bool bf16, const float *M0,
                              const float *Minit, const float *dy, const float *dMT,
                              const float *alpha, const float *beta, float *dkp, float *dqp,
                              float *dv, float *dalpha, float *dbeta, float *dMinit, float *dM0,
                              hipStream_t st);

}  // namespace sdm
