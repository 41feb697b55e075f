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

// Nearest bfloat16 (ties to even) of a finite float, as its 16 bits.
__device__ __forceinline__ uint32_t bf16_bits(float f)
{
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
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
    bool state_bf16;
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

// M[b] <- M0 for every sequence b.
hipError_t launch_init(const Shape &s, const float *M0, void *M, bool state_bf16, hipStream_t st);

// Adds forwarding codes (distance < depth) to the slot words of all records.
hipError_t launch_plan(const Shape &s, uint32_t *rec, int depth, hipStream_t st);

// Token-serial write/read over the records (float4 path): needs d_v % 4 == 0
// and one chain's state within 2^31 bytes.
bool rw_serial_supported(const Shape &s);
hipError_t launch_rw_serial(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st);
int rw_serial_depth();  // prefetch depth the serial kernel is compiled for

// Token-serial write/read, one column per lane, no prefetch (any d_v).
hipError_t launch_rw_simple(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, float *M, hipStream_t st);

// Time-parallel schedule (epochs of tokens, slot-sorted write events).
bool tp_supported(const Shape &s);
int tp_epoch_len(const Shape &s);
size_t tp_workspace_bytes(const Shape &s);  // beyond the token records
// Epochs [ep0, ep1) (ep1 < 0: through the last epoch).
hipError_t launch_tp_prepare(const Shape &s, const uint32_t *rec, void *ws, hipStream_t st,
                             int ep0 = 0, int ep1 = -1, bool link = true);
hipError_t launch_tp_apply(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                           bool bf16, float *y, void *M, bool state_bf16, hipStream_t st,
                           int ep0 = 0, int ep1 = -1);

// One-token step (T == 1): the token's writes, then its reads, in one kernel
// (d_v % 4 == 0 and one chain's state within 2^31 bytes).
bool decode_supported(const Shape &s);
hipError_t launch_rw_decode(const Shape &s, const uint32_t *rec, const void *v, bool bf16,
                            float *y, void *M, bool state_bf16, hipStream_t st);

// Backward (float32 state): a forward write pass that records, per write
// event, the row it replaced ([chain][T][W][d_v]); the write and read events
// of every epoch sorted together by slot; the reverse pass.
hipError_t launch_tp_forward_tape(const Shape &s, const uint32_t *rec, void *ws, const void *v,
                                  bool bf16, float *M, float *tape, hipStream_t st);
hipError_t launch_tp_sort_merged(const Shape &s, const uint32_t *rec, void *ws, TPEntry *out,
                                 uint64_t *tmpA, uint64_t *tmpB, hipStream_t st);
size_t tp_backward_workspace_bytes(const Shape &s);  // beyond the forward's workspace
hipError_t launch_tp_backward(const Shape &s, const uint32_t *rec, void *fwd_ws, void *bwd_ws,
                              const void *v, bool bf16, const float *M0, const float *Minit,
                              const float *dy, const float *dMT, const float *alpha,
                              const float *beta, float *dkp, float *dqp, float *dv, float *dalpha,
                              float *dbeta, float *dMinit, float *dM0, hipStream_t st);

}  // namespace sdm
