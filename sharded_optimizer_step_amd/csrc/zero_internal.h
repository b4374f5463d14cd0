// zero_internal.h -- types shared by the host library and the gfx950 kernels
// of the per-rank ZeRO shard step. Not part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>

#include "zero_step.h"

namespace zero {

constexpr int kThreads = 256;                // one workgroup = 4 wave64
constexpr int kVec = 8;                      // elements per vector: 16 B of bf16, 32 B of fp32
constexpr int kTileElems = kThreads * kVec;  // 2048 elements per tile
constexpr int kInlineRanks = 64;             // rank pointers passed by value per reduce pass
constexpr int kMaxPartials = 8192;           // per-workgroup partial records of one launch
constexpr size_t kAlign = 256;
// Bytes of the per-device static workspace of zero_step_noalloc (64 MiB).
constexpr size_t kScratchBytes = size_t(64) << 20;
constexpr int kMaxDevices = 64;  // devices whose static workspace address is kept

// binary64 scalars of one AdamW step, derived on the host.
struct AdamScalars {
    double b1, omb1, b2, omb2;  // beta1, 1-beta1, beta2, 1-beta2
    double decay;               // 1 - lr*weight_decay
    double lr;
    double bc1, bc2;            // 1 - beta1^t, 1 - beta2^t
    double eps;
};

// How the elements of one shard are visited.
//   vector mode (nvec >= 0): [0, head) one by one, then nvec 16-byte vectors of
//     8 elements, then `tail` elements one by one; every pointer of the shard
//     is 16-byte aligned at element `head`.
//   scalar mode (nvec < 0): every element one by one (pointers that disagree
//     on their alignment modulo 16 bytes).
struct Layout {
    int64_t n;
    int64_t nvec;
    int32_t head;
    int32_t tail;
};

// Tiles of `tile_vecs` vectors (8 elements each) covering one shard.
__host__ __device__ inline int64_t layout_tiles(const Layout& L, int64_t tile_vecs = kThreads)
{
    if (L.n <= 0) return 0;
    if (L.nvec >= 0) {
        const int64_t t = (L.nvec + tile_vecs - 1) / tile_vecs;
        return t > 0 ? t : 1;
    }
    const int64_t te = tile_vecs * kVec;
    return (L.n + te - 1) / te;
}

// Geometry of the fused kernels: NT threads per workgroup, U vectors per
// thread per tile. Within a tile, thread (wave w, lane l) owns vectors
// w*64*U + u*64 + l (u < U): each load instruction of a wave reads 1 KiB
// contiguous, and the workgroup reads NT*U*16 contiguous bytes of one replica
// before any wave moves on to the next replica.
struct Geom {
    int nt;
    int u;
};
constexpr Geom kGeoms[] = {{256, 1}, {1024, 1}, {1024, 2}, {1024, 4}, {1024, 8}, {512, 16}, {256, 16}};
constexpr int kNumGeoms = sizeof(kGeoms) / sizeof(kGeoms[0]);

// Upper bound of layout_tiles over every alignment of an n-element shard.
__host__ __device__ inline int64_t tiles_bound(int64_t n) { return n <= 0 ? 0 : (n + kTileElems - 1) / kTileElems + 1; }

// One tensor of a zero_step plan, as stored in the workspace.
struct alignas(16) TensorDesc {
    const uint16_t* const* grads;  // device address of this tensor's M rank pointers
    float* master;
    float* exp_avg;
    float* exp_avg_sq;
    uint16_t* out;
    float* gbuf;                   // fp32 reduced gradient (two-pass plans), or null
    int64_t n;
    int64_t nvec;
    int32_t head;
    int32_t tail;
    int64_t tile_begin[2];         // first tile of this tensor in the fold-pass / update-pass maps
    int64_t ntiles[2];
};
static_assert(sizeof(TensorDesc) == 112, "TensorDesc layout");

struct TileRef {
    int32_t tensor;
    int32_t local;  // tile index within the tensor
};

struct alignas(16) Partial {
    double sumsq;
    uint32_t bad;
    uint32_t pad;
};

struct alignas(16) PlanHeader {
    uint64_t signature;
    int64_t tiles[2];  // tiles of the fold pass (one partial each) and of the update pass
    int32_t T;
    int32_t M;
    int32_t geom[2];   // kGeoms index of each pass
    int32_t two_pass;
    int32_t kind;      // PlanKind
};

// What a workspace plan drives: the fused step (one or two passes), the
// accumulation of one gradient bucket, or the step from accumulated gradients.
enum class PlanKind : int32_t { Step = 0, StepTwoPass = 1, Bucket = 2, AccStep = 3, Fold = 4, BucketStep = 5 };

// Byte offset, in the 256-byte header region of a zero_step workspace, of the
// arrival counter of the fold pass (zero between launches).
constexpr size_t kCounterOffset = 128;
// Byte offset, in the same region, of the device result record that a
// fold-only plan (the CPU-offloaded step) writes.
constexpr size_t kRecordOffset = 192;

// What the last workgroup of a fold pass needs to write the result record
// and, in the AMP form (ls non-null), to move the loss scale.
struct FinalizeArgs {
    zero_result* res;
    unsigned* counter;
    double external;
    double max_norm;
    int skip;
    zero_loss_scale* ls;           // non-null (AMP): the fold's last workgroup moves this loss scale
    zero_loss_scale_config lscfg;  // meaningful when ls is non-null
    const zero_loss_scale* scale_from;  // non-null (AMP): the multiplier is gscale * scale_from->inv_scale
    // bucket accumulation (Mode::Acc): the last workgroup of a final pass
    // writes the bucket partial instead of a result record
    zero_bucket_partial* slot;
    uint64_t stamp;
    int accumulate;                // add the fold to the accumulator
    int final;                     // last micro-batch: norm partials into *slot
    int stream;                    // the single pass's state stores stream past the caches (stream_state_stores)
};

// The Infinity Cache of an MI355X (256 MiB) takes a step's state writes and
// writes them back later. When a step writes more than it holds, those
// write-backs fall among the step's own reads, and state stores that go out to
// memory as they are written are faster; when the writes fit, keeping them is
// faster. The choice is made per step from what it writes: 12 bytes of state
// and 2 of bf16 output per parameter.
inline bool stream_state_stores(int64_t n) { return n > ZERO_STREAM_STORES_MIN_PARAMS; }

// Byte offsets of the regions of a zero_step workspace.
struct PlanOffsets {
    size_t desc, ptrs, map0, map1, parts, gbuf, total;
};

// Payload of one plan-upload launch (carried in the kernel arguments).
constexpr int kWriteWords = 500;
struct WriteChunk {
    uint64_t offset;  // byte offset in the workspace, 4-byte aligned
    uint32_t words;
    uint32_t pad;
    uint32_t data[kWriteWords];
};

// Rank pointers passed by value to the flat reduce kernel.
struct RankPtrs {
    const uint16_t* p[kInlineRanks];
};

enum class Mode : int {
    Full = 0,   // fold + unscale + check + AdamW + emit, one pass
    PassA = 1,  // fold + unscale + check, store fp32 g
    PassB = 2,  // read fp32 g, times gscale, AdamW + emit (coefficient/skip from the result record)
    Acc = 3,    // fold into the fp32 accumulator; on the final pass, check + norm partials
    BucketFull = 4,  // Full for a ZeRO-2 bucket's final micro-batch: g = (acc + fold or fold) * gscale, AdamW +
                     // emit, norm partials into the bucket partial (no clipping, no skipping)
};

// ---- launch wrappers (zero_kernels.hip); all return a hipError_t ----------

hipError_t launch_reduce(const RankPtrs& ptrs, int Mc, bool first, bool last, float scale, const Layout& L,
                         float* g_out, int grid, hipStream_t s);
hipError_t launch_check(const float* g, const Layout& L, Partial* parts, int grid, hipStream_t s);
hipError_t launch_adamw(float* master, float* m, float* v, const float* g, uint16_t* out, const Layout& L,
                        const AdamScalars& c, const zero_result* res, int grid, hipStream_t s);
// Norm/flag finalize of the composed entry points: nparts partials combined
// in index order into the result record.
hipError_t launch_finalize(const Partial* parts, int64_t nparts, double external, double max_norm, int skip,
                           zero_result* res, hipStream_t s);
// The bucket partials of a ZeRO-2 step combined in index order into the
// result record, each checked against the step's stamp and fp32 multiplier
// (scale, times ls->inv_scale when ls is non-null); a stale plan `hdr` (may
// be null) is reported instead.
hipError_t launch_bucket_finalize(const PlanHeader* hdr, uint64_t sig, const zero_bucket_partial* parts, int32_t nb,
                                  uint64_t stamp, float scale, const zero_loss_scale* ls, double external,
                                  double max_norm, int skip, zero_result* res, hipStream_t s);
// The partial of a final bucket pass over no elements (scale times
// ls->inv_scale when ls is non-null).
hipError_t launch_bucket_partial_empty(zero_bucket_partial* slot, uint64_t stamp, float scale,
                                       const zero_loss_scale* ls, hipStream_t s);
hipError_t launch_loss_scale_init(const zero_loss_scale& s, zero_loss_scale* ls, hipStream_t st);
hipError_t launch_loss_scale_update(const zero_loss_scale_config& c, const zero_result* res, zero_loss_scale* ls,
                                    hipStream_t st);
hipError_t launch_plan_write(uint8_t* ws, const WriteChunk& c, hipStream_t s);
hipError_t launch_plan_tiles(const TensorDesc* desc, int T, TileRef* map0, TileRef* map1, hipStream_t s);
// One workgroup per tile: grid = tiles of the pass. The fold passes (Full,
// PassA) also finalize: their last workgroup writes the result record `fin`.
// The update pass (PassB) reads coef and skip from `res`.
hipError_t launch_fused(Mode mode, int geom, const PlanHeader* hdr, const TensorDesc* desc, const TileRef* map,
                        int64_t tiles, uint64_t sig, int M, float gscale, const AdamScalars& c, Partial* parts,
                        const FinalizeArgs& fin, const zero_result* res, hipStream_t s);

// Workgroups of 256 threads that one kernel keeps resident on the current
// device (occupancy x compute units), for the grid-stride launches.
int resident_grid_reduce(int Mc, bool first);
int resident_grid_check();
int resident_grid_adamw();
int compute_units();  // of the current device
// Device address of the current device's static workspace (kScratchBytes,
// 256-byte aligned), resolved on the first call on each device.
hipError_t scratch_workspace(void** ptr);

}  // namespace zero
