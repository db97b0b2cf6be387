// C ABI of libssm: argument validation on the host, plan selection, kernel launches.
// Every check runs before anything is enqueued and without touching the device, so invalid
// calls fail the same way on a machine with no GPU.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/ssm.h"
#include "kernels.h"

// Scratch of ssm_scan_fwd_noalloc (the segment carries of a long, narrow input): a file-scope
// device array, one copy per GPU, alive until the process ends. In host code this name is a
// host-side stand-in, never a device address: host code uses only the address that
// hipGetSymbolAddress returned for the current device (scratch_for_current_device below).
constexpr size_t kNoallocScratchBytes = SSM_SCAN_NOALLOC_SCRATCH_BYTES;
__device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {

thread_local std::string g_detail;

ssm_status fail(ssm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_detail = buf;
  return s;
}

ssm_status ok() {
  g_detail.clear();
  return SSM_OK;
}

ssm_status from_hip(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(SSM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device address of `scratch` on the current device, looked up once per device (with that device
// current) and kept: each GPU holds its own copy of the array at its own address.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

ssm_status scratch_for_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return from_hip(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(SSM_ERR_UNSUPPORTED, "device %d: the static scratch supports devices 0..%d", dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return from_hip(e, "hipGetSymbolAddress(scratch)");
    if (!ptr) return fail(SSM_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SSM_OK;
}

// The bits of an enum argument as an int. A C caller may pass any value, and reading an
// out-of-range value as the C++ enum type is undefined, so entry points take the bits first.
template <typename E>
int enum_bits(const E& e) {
  static_assert(sizeof(E) == sizeof(int), "C enums are int-sized");
  int v;
  std::memcpy(&v, &e, sizeof v);
  return v;
}

size_t io_size(int t) { return t == SSM_BF16 ? 2 : 4; }

bool valid_dtype(int t) { return t == SSM_F32 || t == SSM_BF16; }

// [p, p + bytes) overlaps [q, q + qbytes)?
bool overlaps(const void* p, size_t bytes, const void* q, size_t qbytes) {
  if (!p || !q || bytes == 0 || qbytes == 0) return false;
  const uintptr_t a = reinterpret_cast<uintptr_t>(p), b = reinterpret_cast<uintptr_t>(q);
  return a < b + qbytes && b < a + bytes;
}

bool supported_scan_n(int64_t N) { return N == 1 || N == 2 || N == 4 || N == 8 || N == 16; }

// The library targets MI355X (256 compute units); the plan depends only on the shapes, so the
// workspace query needs no device.
// The scan kernels address a 16-token tile with 32-bit per-lane byte offsets (16 rows of D
// elements of at most 4 bytes): D up to 2^24 keeps them far below 2^32.
constexpr int64_t kMaxScanD = int64_t(1) << 24;
constexpr int64_t kPlanCUs = 256;
constexpr int64_t kTile = 16;         // tokens per LDS tile of the scan kernels
constexpr int64_t kMinSegment = 256;  // shortest automatic segment

int64_t auto_segment_len(int64_t B, int64_t L, int64_t D, int64_t N) {
  const int64_t ch = ssm::scan_channels_per_tile(N);
  const int64_t wgs = ((D + ch - 1) / ch) * B;
  if (L <= kMinSegment || wgs >= 2 * kPlanCUs) return L;
  // aim for four workgroups per CU (measured on the long, narrow fp32 scan: one round of four
  // per CU, or two, beats one of five, whose segment pass ran slower per token)
  int64_t nseg = (4 * kPlanCUs + wgs - 1) / wgs;
  int64_t seg = (L + nseg - 1) / nseg;
  seg = ((seg + kTile - 1) / kTile) * kTile;
  if (seg < kMinSegment) seg = kMinSegment;
  return seg >= L ? L : seg;
}

int64_t num_segments(int64_t L, int64_t seg_len) { return seg_len >= L ? 1 : (L + seg_len - 1) / seg_len; }

ssm_status scan_common(int64_t B, int64_t L, int64_t D, int64_t N, int io, const void* x,
                       const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                       const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                       void* y, float* h_last, int64_t seg_len, void* ws, size_t ws_bytes, void* stream,
                       int64_t conv_W = 0, const float* conv_w = nullptr, const float* conv_b = nullptr,
                       void* conv_state = nullptr, bool static_scratch = false) {
  if (B < 0 || L < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "B=%lld and L=%lld must be >= 0", (long long)B, (long long)L);
  if (D < 1 || (D % 4) != 0) return fail(SSM_ERR_INVALID_ARGUMENT, "D=%lld must be >= 1 and a multiple of 4", (long long)D);
  if (!valid_dtype(io)) return fail(SSM_ERR_INVALID_ARGUMENT, "unknown io_dtype %d", (int)io);
  if (!supported_scan_n(N)) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported state sizes are 1, 2, 4, 8, 16", (long long)N);
  if (D > kMaxScanD) return fail(SSM_ERR_UNSUPPORTED, "D=%lld: at most %lld channels", (long long)D, (long long)kMaxScanD);
  if (seg_len < 1) return fail(SSM_ERR_INVALID_ARGUMENT, "segment_len=%lld must be >= 1", (long long)seg_len);
  if (conv_w && (conv_W < 1 || conv_W > 4))
    return fail(SSM_ERR_UNSUPPORTED, "conv_width=%lld: the fused prefill convolution supports 1..4", (long long)conv_W);
  if (conv_w && conv_state && !aligned16(conv_state))
    return fail(SSM_ERR_INVALID_ARGUMENT, "conv_state must be 16-byte aligned");
  if (B == 0) return ok();
  if (!A) return fail(SSM_ERR_INVALID_ARGUMENT, "A is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t stb = (size_t)(B * D * N) * sizeof(float);
  if (h_last && h0 && h_last != h0 && overlaps(h_last, stb, h0, stb))
    return fail(SSM_ERR_INVALID_ARGUMENT, "h_last partially overlaps h0 (it may only equal it)");
  if (L == 0) {
    if (!h_last || h_last == h0) return ok();
    if (static_scratch)   // no memory-set or copy node: a kernel
      return from_hip(ssm::launch_state_fill(h_last, h0, B * D * N, st), "L == 0 state fill");
    hipError_t e = h0 ? hipMemcpyAsync(h_last, h0, stb, hipMemcpyDeviceToDevice, st)
                      : hipMemsetAsync(h_last, 0, stb, st);
    return from_hip(e, "L == 0 state copy");
  }
  if (!x || !delta || !Bm || !Cm || !y)
    return fail(SSM_ERR_INVALID_ARGUMENT, "x, delta, Bm, Cm and y must not be NULL");
  if (!aligned16(x) || !aligned16(delta) || !aligned16(y) || (z && !aligned16(z)) || !aligned16(Bm) || !aligned16(Cm))
    return fail(SSM_ERR_INVALID_ARGUMENT, "per-token tensors must be 16-byte aligned");
  const size_t es = io_size(io);
  const size_t tok = (size_t)(B * L * D) * es, bc = (size_t)(B * L * N) * es;
  const void* ins[] = {x, delta, z, Bm, Cm, A, delta_bias, Dskip, h0};
  const size_t insz[] = {tok, tok, tok, bc, bc, (size_t)(D * N) * 4, (size_t)D * 4, (size_t)D * 4, stb};
  for (int k = 0; k < 9; ++k)
    if (overlaps(y, tok, ins[k], insz[k])) return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps an input");
  if (h_last && overlaps(h_last, stb, y, tok)) return fail(SSM_ERR_INVALID_ARGUMENT, "h_last overlaps y");
  if (conv_w) {
    const size_t reg = (size_t)(B * D * conv_W) * es;
    const void* cins[] = {x, delta, z, Bm, Cm, A, delta_bias, Dskip, h0, h_last, y, conv_w, conv_b};
    const size_t cinsz[] = {tok, tok, tok, bc, bc, (size_t)(D * N) * 4, (size_t)D * 4, (size_t)D * 4, stb, stb,
                            tok, (size_t)(D * conv_W) * 4, (size_t)D * 4};
    for (int k = 0; k < 13; ++k)
      if (overlaps(conv_state, reg, cins[k], cinsz[k]))
        return fail(SSM_ERR_INVALID_ARGUMENT, "conv_state overlaps another tensor");
    if (overlaps(y, tok, conv_w, cinsz[11]) || overlaps(y, tok, conv_b, cinsz[12]))
      return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps an input");
  }

  const int64_t nseg = num_segments(L, seg_len);
  if (B > 65535 || nseg > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "B=%lld and the segment count %lld must each be <= 65535", (long long)B,
                (long long)nseg);
  const size_t need = ssm::scan_workspace_bytes(B, D, N, nseg);
  if (static_scratch && need > 0) {
    if (need > kNoallocScratchBytes)
      return fail(SSM_ERR_WORKSPACE_TOO_SMALL,
                  "the plan for these sizes needs %zu bytes of scratch; the static scratch holds %zu "
                  "(use ssm_scan_fwd with a workspace)", need, kNoallocScratchBytes);
    const ssm_status sc = scratch_for_current_device(&ws);
    if (sc != SSM_OK) return sc;
    ws_bytes = kNoallocScratchBytes;
  }
  if (need > 0) {
    if (!ws) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", need);
    if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
    if (!aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  }
  ssm::ScanParams p{};
  p.B = B; p.L = L; p.D = D; p.N = N;
  p.io_bf16 = io == SSM_BF16;
  p.x = x; p.delta = delta; p.z = z; p.Bm = Bm; p.Cm = Cm;
  p.delta_bias = delta_bias; p.A = A; p.Dskip = Dskip; p.h0 = h0;
  p.y = y; p.h_last = h_last; p.delta_softplus = delta_softplus ? 1 : 0;
  p.nseg = nseg;
  p.seg_len = nseg == 1 ? L : seg_len;
  if (nseg > 1) {
    p.ws_h = static_cast<float*>(ws);
    p.ws_sum = p.ws_h + B * nseg * D * N;
    p.ws_neg = reinterpret_cast<int*>(p.ws_sum + B * nseg * D);
  }
  if (conv_w) {
    p.conv_w = conv_w; p.conv_b = conv_b; p.conv_W = (int)conv_W;
    p.conv_in = conv_state; p.conv_out = conv_state;
  }
  return from_hip(ssm::launch_scan(p, st), "ssm_scan_fwd launch");
}

// Backward plan: the forward's automatic segments (multiples of 16 tokens); an explicit length
// is rounded up to a multiple of 16.
int64_t bwd_segment_len(int64_t L, int64_t seg_len) {
  seg_len = ((seg_len + kTile - 1) / kTile) * kTile;
  return seg_len >= L ? L : seg_len;
}

ssm_status scan_bwd_common(int64_t B, int64_t L, int64_t D, int64_t N, int io, const void* x,
                           const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                           const void* Bm, const void* Cm, const float* Dskip, const void* z,
                           const float* h0, const void* dy, const float* dh_last, void* dx, void* ddelta,
                           float* dA, float* dBm, float* dCm, float* dDskip, float* ddelta_bias, void* dz,
                           float* dh0, int64_t seg_len, void* ws, size_t ws_bytes, void* stream) {
  if (B < 0 || L < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "B=%lld and L=%lld must be >= 0", (long long)B, (long long)L);
  if (D < 1 || (D % 4) != 0) return fail(SSM_ERR_INVALID_ARGUMENT, "D=%lld must be >= 1 and a multiple of 4", (long long)D);
  if (!valid_dtype(io)) return fail(SSM_ERR_INVALID_ARGUMENT, "unknown io_dtype %d", (int)io);
  if (!supported_scan_n(N)) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported state sizes are 1, 2, 4, 8, 16", (long long)N);
  if (D > kMaxScanD) return fail(SSM_ERR_UNSUPPORTED, "D=%lld: at most %lld channels", (long long)D, (long long)kMaxScanD);
  if (seg_len < 1) return fail(SSM_ERR_INVALID_ARGUMENT, "segment_len=%lld must be >= 1", (long long)seg_len);
  if (!A || !dA) return fail(SSM_ERR_INVALID_ARGUMENT, "A and dA must not be NULL");
  if (z && !dz) return fail(SSM_ERR_INVALID_ARGUMENT, "dz must be given with z");
  const size_t es = io_size(io);
  const size_t tok = (size_t)(B * L * D) * es, bc = (size_t)(B * L * N) * es;
  const size_t bcg = (size_t)(B * L * N) * 4, stb = (size_t)(B * D * N) * 4;
  const size_t pd = (size_t)(D * N) * 4, vd = (size_t)D * 4;
  if (B > 0 && L > 0) {
    if (!x || !delta || !Bm || !Cm || !dy || !dx || !ddelta || !dBm || !dCm)
      return fail(SSM_ERR_INVALID_ARGUMENT, "x, delta, Bm, Cm, dy, dx, ddelta, dBm and dCm must not be NULL");
    if (!aligned16(x) || !aligned16(delta) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(dy) ||
        !aligned16(dx) || !aligned16(ddelta) || (z && !aligned16(z)) || (dz && !aligned16(dz)))
      return fail(SSM_ERR_INVALID_ARGUMENT, "per-token tensors must be 16-byte aligned");
  }
  // outputs overlap no input and no other output
  const void* ins[] = {x, delta, z, Bm, Cm, dy, A, delta_bias, Dskip, h0, dh_last};
  const size_t insz[] = {tok, tok, tok, bc, bc, tok, pd, vd, vd, stb, stb};
  void* outs[] = {dx, ddelta, z ? dz : nullptr, dA, dBm, dCm, dDskip, ddelta_bias, dh0};
  const size_t outsz[] = {tok, tok, tok, pd, bcg, bcg, vd, vd, stb};
  for (int o = 0; o < 9; ++o) {
    for (int k = 0; k < 11; ++k)
      if (overlaps(outs[o], outsz[o], ins[k], insz[k]))
        return fail(SSM_ERR_INVALID_ARGUMENT, "a gradient output overlaps an input");
    for (int k = o + 1; k < 9; ++k)
      if (overlaps(outs[o], outsz[o], outs[k], outsz[k]))
        return fail(SSM_ERR_INVALID_ARGUMENT, "two gradient outputs overlap");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B == 0 || L == 0) {
    // empty sums: parameter gradients are zero; dh0 is dh_last passed through (or zero)
    hipError_t e = hipMemsetAsync(dA, 0, pd, st);
    if (e == hipSuccess && dDskip) e = hipMemsetAsync(dDskip, 0, vd, st);
    if (e == hipSuccess && ddelta_bias) e = hipMemsetAsync(ddelta_bias, 0, vd, st);
    if (e == hipSuccess && dh0 && B > 0)
      e = dh_last ? hipMemcpyAsync(dh0, dh_last, stb, hipMemcpyDeviceToDevice, st) : hipMemsetAsync(dh0, 0, stb, st);
    return from_hip(e, "empty backward");
  }
  const int64_t sl = bwd_segment_len(L, seg_len);
  const int64_t nseg = num_segments(L, sl);
  if (B > 65535 || nseg > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "B=%lld and the segment count %lld must each be <= 65535", (long long)B,
                (long long)nseg);
  const size_t need = ssm::scan_bwd_workspace_bytes(B, L, D, N, nseg);
  if (!ws) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", need);
  if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");

  ssm::ScanBwdParams p{};
  p.B = B; p.L = L; p.D = D; p.N = N;
  p.io_bf16 = io == SSM_BF16;
  p.delta_softplus = delta_softplus ? 1 : 0;
  p.x = x; p.delta = delta; p.z = z; p.Bm = Bm; p.Cm = Cm; p.dy = dy;
  p.delta_bias = delta_bias; p.A = A; p.Dskip = Dskip; p.h0 = h0; p.dh_last = dh_last;
  p.dx = dx; p.ddelta = ddelta; p.dz = z ? dz : nullptr; p.dA = dA; p.dBm = dBm; p.dCm = dCm;
  p.dDskip = dDskip; p.ddelta_bias = ddelta_bias; p.dh0 = dh0;
  p.seg_len = sl; p.nseg = nseg;
  const int64_t ch = ssm::scan_bwd_channels_per_wg(N);
  p.nct = (D + ch - 1) / ch;
  ssm::scan_bwd_workspace_carve(p, ws);
  return from_hip(ssm::launch_scan_bwd(p, st), "ssm_scan_bwd launch");
}

// Heads per workgroup in the SSD backward's main pass: a divisor of the heads per group (the
// workgroup's heads share the staged B, C and C B^T of the chunk, and their dB and dC are summed
// in registers before one partial per workgroup is written). At least the largest divisor up to
// 4, then the largest one up to 64 that still leaves four workgroups per compute unit of a
// 256-CU device: at 80 heads, L = 8192, B = 2 that is 20 (4, 16, 20 and 40 measured 1.93, 1.80,
// 1.79 and 1.78 ms for the whole backward).
int64_t ssd_bwd_heads_per_wg(int64_t B, int64_t L, int64_t H, int64_t G) {
  const int64_t hg = H / G, nch = (L + ssm::kSsdBwdQ - 1) / ssm::kSsdBwdQ;
  int64_t best = 1;
  for (int64_t hb = 2; hb <= hg && hb <= 64; ++hb)
    if (hg % hb == 0 && (hb <= 4 || (H / hb) * nch * B >= 4 * 256)) best = hb;
  return best;
}

}  // namespace

extern "C" {

int ssm_abi_version(void) { return SSM_ABI_VERSION; }

const char* ssm_status_string(ssm_status status) {
  // A C caller may pass any int; its bytes are read as an int (reading an out-of-range value as
  // the enum type would be undefined in C++).
  int s;
  std::memcpy(&s, &status, sizeof s);
  switch (s) {
    case SSM_OK: return "SSM_OK";
    case SSM_ERR_INVALID_ARGUMENT: return "SSM_ERR_INVALID_ARGUMENT";
    case SSM_ERR_UNSUPPORTED: return "SSM_ERR_UNSUPPORTED";
    case SSM_ERR_WORKSPACE_TOO_SMALL: return "SSM_ERR_WORKSPACE_TOO_SMALL";
    case SSM_ERR_HIP: return "SSM_ERR_HIP";
  }
  return "SSM_ERR_UNKNOWN";
}

const char* ssm_last_error_detail(void) { return g_detail.c_str(); }

size_t ssm_scan_fwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0) return 0;
  return ssm::scan_workspace_bytes(B, D, N, num_segments(L, auto_segment_len(B, L, D, N)));
}

size_t ssm_scan_fwd_segmented_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t segment_len) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0 || segment_len < 1) return 0;
  return ssm::scan_workspace_bytes(B, D, N, num_segments(L, segment_len));
}

ssm_status ssm_scan_fwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                        const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                        const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                        void* y, float* h_last, void* ws, size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  const int64_t seg = (B > 0 && L > 0 && D > 0) ? auto_segment_len(B, L, D, N) : 1;
  return scan_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, y,
                     h_last, seg, ws, ws_bytes, stream);
}

size_t ssm_scan_fwd_conv_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t segment_len) {
  if (B <= 0 || L <= 0 || D <= 0 || N <= 0 || segment_len < 0) return 0;
  int64_t seg = auto_segment_len(B, L, D, N);
  if (segment_len > 0) seg = segment_len >= L ? L : ((segment_len + kTile - 1) / kTile) * kTile;
  return ssm::scan_workspace_bytes(B, D, N, num_segments(L, seg));
}

ssm_status ssm_scan_fwd_conv(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                             const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                             const void* Bm, const void* Cm, const float* Dskip, const void* z,
                             const float* h0, int64_t conv_width, const float* conv_w, const float* conv_b,
                             void* conv_state, void* y, float* h_last, int64_t segment_len, void* ws,
                             size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  if (!conv_w) return fail(SSM_ERR_INVALID_ARGUMENT, "conv_w is NULL");
  if (segment_len < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "segment_len=%lld must be >= 0", (long long)segment_len);
  // segments must start on 16-token tiles (the convolution reads the three rows before a tile)
  int64_t seg = (B > 0 && L > 0 && D > 0) ? auto_segment_len(B, L, D, N) : 1;
  if (segment_len > 0) seg = segment_len >= L ? L : ((segment_len + kTile - 1) / kTile) * kTile;
  return scan_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, y,
                     h_last, seg, ws, ws_bytes, stream, conv_width, conv_w, conv_b, conv_state);
}

ssm_status ssm_scan_fwd_noalloc(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                                const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                                const void* Bm, const void* Cm, const float* Dskip, const void* z,
                                const float* h0, void* y, float* h_last, void* stream) {
  const int io = enum_bits(io_arg);
  const int64_t seg = (B > 0 && L > 0 && D > 0) ? auto_segment_len(B, L, D, N) : 1;
  return scan_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, y, h_last,
                     seg, nullptr, 0, stream, 0, nullptr, nullptr, nullptr, true);
}

ssm_status ssm_scan_fwd_segmented(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                                  const void* delta, const float* delta_bias, int delta_softplus,
                                  const float* A, const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* h0, void* y, float* h_last, int64_t segment_len,
                                  void* ws, size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  return scan_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, y,
                     h_last, segment_len, ws, ws_bytes, stream);
}

size_t ssm_scan_bwd_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype) {
  if (B <= 0 || L <= 0 || D <= 0 || !supported_scan_n(N)) return 0;
  const int64_t sl = bwd_segment_len(L, auto_segment_len(B, L, D, N));
  return ssm::scan_bwd_workspace_bytes(B, L, D, N, num_segments(L, sl));
}

size_t ssm_scan_bwd_segmented_workspace_bytes(int64_t B, int64_t L, int64_t D, int64_t N, int64_t segment_len) {
  if (B <= 0 || L <= 0 || D <= 0 || !supported_scan_n(N) || segment_len < 1) return 0;
  const int64_t sl = bwd_segment_len(L, segment_len);
  return ssm::scan_bwd_workspace_bytes(B, L, D, N, num_segments(L, sl));
}

ssm_status ssm_scan_bwd(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                        const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                        const void* Bm, const void* Cm, const float* Dskip, const void* z, const float* h0,
                        const void* dy, const float* dh_last, void* dx, void* ddelta, float* dA, float* dBm,
                        float* dCm, float* dDskip, float* ddelta_bias, void* dz, float* dh0, void* ws,
                        size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  const int64_t seg = (B > 0 && L > 0 && D > 0) ? auto_segment_len(B, L, D, N) : 1;
  return scan_bwd_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, dy,
                         dh_last, dx, ddelta, dA, dBm, dCm, dDskip, ddelta_bias, dz, dh0, seg, ws, ws_bytes,
                         stream);
}

ssm_status ssm_scan_bwd_segmented(int64_t B, int64_t L, int64_t D, int64_t N, ssm_dtype io_arg, const void* x,
                                  const void* delta, const float* delta_bias, int delta_softplus,
                                  const float* A, const void* Bm, const void* Cm, const float* Dskip,
                                  const void* z, const float* h0, const void* dy, const float* dh_last,
                                  void* dx, void* ddelta, float* dA, float* dBm, float* dCm, float* dDskip,
                                  float* ddelta_bias, void* dz, float* dh0, int64_t segment_len, void* ws,
                                  size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  return scan_bwd_common(B, L, D, N, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm, Dskip, z, h0, dy,
                         dh_last, dx, ddelta, dA, dBm, dCm, dDskip, ddelta_bias, dz, dh0, segment_len, ws,
                         ws_bytes, stream);
}

ssm_status ssm_state_update(int64_t B, int64_t D, int64_t N, int64_t W, ssm_dtype io_arg, const void* x,
                            const void* delta, const float* delta_bias, int delta_softplus, const float* A,
                            const void* Bm, const void* Cm, const float* Dskip, const void* z,
                            void* conv_state, const float* conv_w, const float* conv_b, float* h, void* y,
                            void* stream) {
  const int io = enum_bits(io_arg);
  if (B < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "B=%lld must be >= 0", (long long)B);
  if (D < 1) return fail(SSM_ERR_INVALID_ARGUMENT, "D=%lld must be >= 1", (long long)D);
  if (!valid_dtype(io)) return fail(SSM_ERR_INVALID_ARGUMENT, "unknown io_dtype %d", (int)io);
  if (!supported_scan_n(N)) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported state sizes are 1, 2, 4, 8, 16", (long long)N);
  if (conv_state && (W < 1 || W > 8)) return fail(SSM_ERR_UNSUPPORTED, "conv_width=%lld: supported 1..8", (long long)W);
  if (B == 0) return ok();
  if (!x || !delta || !A || !Bm || !Cm || !h || !y)
    return fail(SSM_ERR_INVALID_ARGUMENT, "x, delta, A, Bm, Cm, h and y must not be NULL");
  if (conv_state && !conv_w) return fail(SSM_ERR_INVALID_ARGUMENT, "conv_w is NULL while conv_state is given");
  if (!aligned16(h) || !aligned16(x) || !aligned16(delta) || !aligned16(y) || !aligned16(A) ||
      !aligned16(Bm) || !aligned16(Cm) || (z && !aligned16(z)) ||
      (conv_state && (!aligned16(conv_state) || !aligned16(conv_w))))
    return fail(SSM_ERR_INVALID_ARGUMENT,
                "h, x, delta, z, Bm, Cm, y, A, conv_state and conv_w must be 16-byte aligned");
  const size_t es = io_size(io), tok = (size_t)(B * D) * es;
  const size_t stb = (size_t)(B * D * N) * 4;
  const void* ins[] = {x, delta, z, Bm, Cm, A, h, conv_state, conv_w};
  const size_t insz[] = {tok, tok, tok, (size_t)(B * N) * es, (size_t)(B * N) * es, (size_t)(D * N) * 4, stb,
                         (size_t)(B * D * (W > 0 ? W : 1)) * es, (size_t)(D * (W > 0 ? W : 1)) * 4};
  for (int k = 0; k < 9; ++k)
    if (overlaps(y, tok, ins[k], insz[k])) return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps an input");
  ssm::StepParams p{};
  p.B = B; p.D = D; p.N = N; p.W = conv_state ? W : 0;
  p.io_bf16 = io == SSM_BF16;
  p.x = x; p.delta = delta; p.z = z; p.Bm = Bm; p.Cm = Cm;
  p.delta_bias = delta_bias; p.A = A; p.Dskip = Dskip;
  p.conv_state = conv_state; p.conv_w = conv_w; p.conv_b = conv_b;
  p.h = h; p.y = y; p.delta_softplus = delta_softplus ? 1 : 0;
  return from_hip(ssm::launch_state_update(p, static_cast<hipStream_t>(stream)), "ssm_state_update launch");
}

size_t ssd_chunk_fwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t chunk,
                                     ssm_dtype io) {
  if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || chunk <= 0) return 0;
  return ssm::ssd_workspace_bytes(B, L, H, P, N, 1, chunk, enum_bits(io) == SSM_F32);
}

size_t ssd_chunk_fwd_grouped_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                                             int64_t chunk, ssm_dtype io) {
  if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || chunk <= 0) return 0;
  return ssm::ssd_workspace_bytes(B, L, H, P, N, G, chunk, enum_bits(io) == SSM_F32);
}

size_t ssm_linear_workspace_bytes(int64_t M, int64_t K, int64_t Nout) {
  if (M <= 0 || K <= 0 || Nout <= 0) return 0;
  return ssm::gemm_workspace_bytes(M, K, Nout);
}

ssm_status ssm_linear(int64_t M, int64_t K, int64_t Nout, const void* x, const void* w, const void* residual, void* y,
                      void* ws, size_t ws_bytes, void* stream) {
  if (M < 0 || M > 128) return fail(SSM_ERR_UNSUPPORTED, "M=%lld: 0..128 token rows", (long long)M);
  if (K < 128 || K % 128 != 0) return fail(SSM_ERR_UNSUPPORTED, "K=%lld must be a positive multiple of 128", (long long)K);
  if (Nout < 4 || Nout % 4 != 0) return fail(SSM_ERR_UNSUPPORTED, "Nout=%lld must be a positive multiple of 4", (long long)Nout);
  if ((Nout + 31) / 32 > 2147483647LL) return fail(SSM_ERR_UNSUPPORTED, "Nout too large");
  if (M == 0) return ok();
  if (!x || !w || !y) return fail(SSM_ERR_INVALID_ARGUMENT, "x, w and y must not be NULL");
  if (!aligned16(x) || !aligned16(w) || !aligned16(y) || (residual && !aligned16(residual)))
    return fail(SSM_ERR_INVALID_ARGUMENT, "x, w, y and residual must be 16-byte aligned");
  const size_t xb = (size_t)(M * K) * 2, wb = (size_t)(Nout * K) * 2, yb = (size_t)(M * Nout) * 2;
  if (overlaps(y, yb, x, xb) || overlaps(y, yb, w, wb))
    return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps x or w");
  if (residual && residual != y && overlaps(residual, yb, y, yb))
    return fail(SSM_ERR_INVALID_ARGUMENT, "residual partially overlaps y (it may only equal it)");
  const size_t need = ssm::gemm_workspace_bytes(M, K, Nout);
  if (need && (!ws || ws_bytes < need))
    return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0, need);
  if (need && !aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  ssm::GemmParams g{};
  g.M = M; g.K = K; g.Nout = Nout; g.x = x; g.ldx = K; g.w = w; g.y = y; g.ldy = Nout; g.residual = residual;
  g.partial = static_cast<float*>(ws);
  return from_hip(ssm::launch_gemm(g, static_cast<hipStream_t>(stream)), "ssm_linear launch");
}

ssm_status ssm_layernorm(int64_t M, int64_t D, const void* x, const float* w, const float* b, float eps, void* y,
                         void* stream) {
  if (M < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "M=%lld must be >= 0", (long long)M);
  if (D < 8 || D % 8 != 0 || D > 8192) return fail(SSM_ERR_UNSUPPORTED, "D=%lld: a multiple of 8 up to 8192", (long long)D);
  if (!(eps > 0.f)) return fail(SSM_ERR_INVALID_ARGUMENT, "eps must be > 0");
  if (M == 0) return ok();
  if (M > 2147483647LL) return fail(SSM_ERR_UNSUPPORTED, "M too large");
  if (!x || !w || !b || !y) return fail(SSM_ERR_INVALID_ARGUMENT, "x, w, b and y must not be NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(SSM_ERR_INVALID_ARGUMENT, "x and y must be 16-byte aligned");
  const size_t rb = (size_t)(M * D) * 2;
  if (y != x && overlaps(y, rb, x, rb)) return fail(SSM_ERR_INVALID_ARGUMENT, "y partially overlaps x (it may only equal it)");
  return from_hip(ssm::launch_layernorm(M, D, x, w, b, eps, y, static_cast<hipStream_t>(stream)), "ssm_layernorm launch");
}

size_t ssm_block_step_workspace_bytes(int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t W, int64_t R) {
  if (B <= 0 || d_model <= 0 || d_inner <= 0 || N <= 0 || W <= 0 || R <= 0) return 0;
  return ssm::block_workspace_bytes(B, d_model, d_inner, N, R);
}

ssm_status ssm_block_step(int64_t B, int64_t d_model, int64_t d_inner, int64_t N, int64_t W, int64_t R, void* hidden,
                          const float* ln_w, const float* ln_b, float eps, const void* W_in, const float* conv_w,
                          const float* conv_b, const void* W_xp, const void* W_dt, const float* b_dt, const float* A,
                          const float* Dskip, const void* W_out, void* conv_state, float* h, void* ws, size_t ws_bytes,
                          void* stream) {
  if (B < 0 || B > 128) return fail(SSM_ERR_UNSUPPORTED, "B=%lld: 0..128 sequences", (long long)B);
  if (d_model < 128 || d_model % 128 != 0 || d_model > 8192)
    return fail(SSM_ERR_UNSUPPORTED, "d_model=%lld: a multiple of 128 up to 8192", (long long)d_model);
  if (d_inner < 128 || d_inner % 128 != 0) return fail(SSM_ERR_UNSUPPORTED, "d_inner=%lld: a multiple of 128", (long long)d_inner);
  if (R < 128 || R % 128 != 0) return fail(SSM_ERR_UNSUPPORTED, "R=%lld: a multiple of 128", (long long)R);
  if (N != 4 && N != 8 && N != 16) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported 4, 8, 16", (long long)N);
  if (W < 1 || W > 8) return fail(SSM_ERR_UNSUPPORTED, "W=%lld: supported 1..8", (long long)W);
  if (!(eps > 0.f)) return fail(SSM_ERR_INVALID_ARGUMENT, "eps must be > 0");
  if (B == 0) return ok();
  const void* need_ptrs[] = {hidden, ln_w, ln_b, W_in, conv_w, W_xp, W_dt, b_dt, A, W_out, conv_state, h};
  for (const void* q : need_ptrs)
    if (!q) return fail(SSM_ERR_INVALID_ARGUMENT, "a required pointer is NULL (only conv_b and Dskip may be)");
  const void* al[] = {hidden, W_in, W_xp, W_dt, W_out, conv_state, h, A};
  for (const void* q : al)
    if (!aligned16(q)) return fail(SSM_ERR_INVALID_ARGUMENT, "hidden, the weight matrices, A, conv_state and h must be 16-byte aligned");
  // the in/out tensors overlap nothing else
  const size_t hb = (size_t)(B * d_model) * 2, cb = (size_t)(B * d_inner * W) * 2, sb = (size_t)(B * d_inner * N) * 4;
  const void* ins[] = {ln_w, ln_b, W_in, conv_w, conv_b, W_xp, W_dt, b_dt, A, Dskip, W_out};
  const size_t insz[] = {(size_t)d_model * 4, (size_t)d_model * 4, (size_t)(2 * d_inner * d_model) * 2,
                         (size_t)(d_inner * W) * 4, (size_t)d_inner * 4, (size_t)((R + 2 * N) * d_inner) * 2,
                         (size_t)(d_inner * R) * 2, (size_t)d_inner * 4, (size_t)(d_inner * N) * 4, (size_t)d_inner * 4,
                         (size_t)(d_model * d_inner) * 2};
  void* io[] = {hidden, conv_state, h};
  const size_t iosz[] = {hb, cb, sb};
  for (int o = 0; o < 3; ++o) {
    for (int k = 0; k < 11; ++k)
      if (overlaps(io[o], iosz[o], ins[k], insz[k])) return fail(SSM_ERR_INVALID_ARGUMENT, "hidden, conv_state or h overlaps a weight");
    for (int k = o + 1; k < 3; ++k)
      if (overlaps(io[o], iosz[o], io[k], iosz[k])) return fail(SSM_ERR_INVALID_ARGUMENT, "hidden, conv_state and h overlap");
  }
  const size_t need = ssm::block_workspace_bytes(B, d_model, d_inner, N, R);
  if (!ws) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", need);
  if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  for (int o = 0; o < 3; ++o)
    if (overlaps(ws, need, io[o], iosz[o])) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps hidden, conv_state or h");
  ssm::BlockParams p{};
  p.B = B; p.Dm = d_model; p.Di = d_inner; p.N = N; p.W = W; p.R = R; p.eps = eps;
  p.hidden = hidden; p.ln_w = ln_w; p.ln_b = ln_b; p.W_in = W_in; p.conv_w = conv_w; p.conv_b = conv_b;
  p.W_xp = W_xp; p.W_dt = W_dt; p.b_dt = b_dt; p.A = A; p.Dskip = Dskip;
  p.W_out = W_out; p.conv_state = conv_state; p.h = h;
  return from_hip(ssm::launch_block_step(p, ws, static_cast<hipStream_t>(stream)), "ssm_block_step launch");
}

size_t ssd_chunk_bwd_workspace_bytes(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, ssm_dtype) {
  if (B <= 0 || L <= 0 || H <= 0 || P <= 0 || N <= 0 || G <= 0 || H % G != 0) return 0;
  return ssm::ssd_bwd_workspace_bytes(B, L, H, P, N, G, ssd_bwd_heads_per_wg(B, L, H, G));
}

}  // extern "C"

namespace {

ssm_status ssd_common(const char* fn, int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G,
                      int64_t chunk, int io, const void* x, const void* delta, const float* delta_bias,
                      int delta_softplus, const float* A, const void* Bm, const void* Cm, const float* Dskip,
                      int dskip_per_channel, const void* z, const float* h0, void* y, float* h_last, void* ws,
                      size_t ws_bytes, void* stream) {
  if (B < 0 || L < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "B and L must be >= 0");
  if (H < 1) return fail(SSM_ERR_INVALID_ARGUMENT, "H=%lld must be >= 1", (long long)H);
  if (G < 1 || H % G != 0)
    return fail(SSM_ERR_INVALID_ARGUMENT, "G=%lld must be >= 1 and divide H=%lld", (long long)G, (long long)H);
  if (!valid_dtype(io)) return fail(SSM_ERR_INVALID_ARGUMENT, "unknown io_dtype %d", (int)io);
  if (P != 64) return fail(SSM_ERR_UNSUPPORTED, "P=%lld: supported head dim is 64", (long long)P);
  if (N != 64 && N != 128) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported 64, 128", (long long)N);
  if (chunk != 64 && chunk != 128 && chunk != 256)
    return fail(SSM_ERR_UNSUPPORTED, "chunk=%lld: supported 64, 128, 256", (long long)chunk);
  const bool f32 = io == SSM_F32;
  const size_t esz = f32 ? 4 : 2;
  // grid limits: chunks and batch rows x groups index grid dimensions y and z, heads x
  if ((L + chunk - 1) / chunk > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "L=%lld: at most 65535 chunks of %lld tokens", (long long)L, (long long)chunk);
  if (B * G > 65535 || H > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "B*G=%lld and H=%lld must each be <= 65535", (long long)(B * G), (long long)H);
  if (B == 0) return ok();
  if (!A) return fail(SSM_ERR_INVALID_ARGUMENT, "A is NULL");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const size_t stb = (size_t)(B * H * P * N) * 4;
  if (h_last && h0 && h_last != h0 && overlaps(h_last, stb, h0, stb))
    return fail(SSM_ERR_INVALID_ARGUMENT, "h_last partially overlaps h0 (it may only equal it)");
  if (L == 0) {
    if (!h_last || h_last == h0) return ok();
    hipError_t e = h0 ? hipMemcpyAsync(h_last, h0, stb, hipMemcpyDeviceToDevice, st) : hipMemsetAsync(h_last, 0, stb, st);
    return from_hip(e, "L == 0 state copy");
  }
  if (!x || !delta || !Bm || !Cm || !y) return fail(SSM_ERR_INVALID_ARGUMENT, "x, delta, Bm, Cm and y must not be NULL");
  if (!aligned16(x) || !aligned16(y) || !aligned16(Bm) || !aligned16(Cm) || (z && !aligned16(z)) ||
      (Dskip && dskip_per_channel && !aligned16(Dskip)))
    return fail(SSM_ERR_INVALID_ARGUMENT, "per-token tensors and a per-channel Dskip must be 16-byte aligned");
  const size_t tok = (size_t)(B * L * H * P) * esz;
  const size_t bc = (size_t)(B * L * G * N) * esz;
  const void* ins[] = {x, delta, z, Bm, Cm, A, h0};
  const size_t insz[] = {tok, (size_t)(B * L * H) * esz, tok, bc, bc, (size_t)H * 4, stb};
  for (int k = 0; k < 7; ++k)
    if (overlaps(y, tok, ins[k], insz[k])) return fail(SSM_ERR_INVALID_ARGUMENT, "y overlaps an input");
  const size_t need = ssm::ssd_workspace_bytes(B, L, H, P, N, G, chunk, f32);
  if (!ws) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", need);
  if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  if (overlaps(ws, need, y, tok)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace overlaps y");
  ssm::SsdParams p{};
  p.B = B; p.L = L; p.H = H; p.P = P; p.N = N; p.Q = chunk; p.G = G;
  p.x = x; p.delta = delta; p.z = z; p.Bm = Bm; p.Cm = Cm;
  p.delta_bias = delta_bias; p.A = A; p.Dskip = Dskip; p.h0 = h0;
  p.dskip_per_channel = Dskip && dskip_per_channel ? 1 : 0;
  p.y = y; p.h_last = h_last; p.delta_softplus = delta_softplus ? 1 : 0;
  p.io_f32 = f32 ? 1 : 0;
  ssm::ssd_workspace_carve(p, ws);
  return from_hip(ssm::launch_ssd(p, st), fn);
}

}  // namespace

extern "C" {

ssm_status ssd_chunk_fwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t chunk, ssm_dtype io_arg,
                         const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                         const float* A, const void* Bm, const void* Cm, const float* Dskip, const void* z,
                         const float* h0, void* y, float* h_last, void* ws, size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  return ssd_common("ssd_chunk_fwd", B, L, H, P, N, 1, chunk, io, x, delta, delta_bias, delta_softplus, A, Bm, Cm,
                    Dskip, 0, z, h0, y, h_last, ws, ws_bytes, stream);
}

ssm_status ssd_chunk_fwd_grouped(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, int64_t chunk,
                                 ssm_dtype io_arg, const void* x, const void* delta, const float* delta_bias,
                                 int delta_softplus, const float* A, const void* Bm, const void* Cm,
                                 const float* Dskip, int dskip_per_channel, const void* z, const float* h0, void* y,
                                 float* h_last, void* ws, size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  return ssd_common("ssd_chunk_fwd_grouped", B, L, H, P, N, G, chunk, io, x, delta, delta_bias, delta_softplus, A,
                    Bm, Cm, Dskip, dskip_per_channel, z, h0, y, h_last, ws, ws_bytes, stream);
}

ssm_status ssd_chunk_bwd(int64_t B, int64_t L, int64_t H, int64_t P, int64_t N, int64_t G, ssm_dtype io_arg,
                         const void* x, const void* delta, const float* delta_bias, int delta_softplus,
                         const float* A, const void* Bm, const void* Cm, const float* Dskip, int dskip_per_channel,
                         const void* z, const float* h0, const void* dy, const float* dh_last, void* dx,
                         void* ddelta, float* dA, float* dBm, float* dCm, float* dDskip, float* ddelta_bias,
                         void* dz, float* dh0, void* ws, size_t ws_bytes, void* stream) {
  const int io = enum_bits(io_arg);
  if (B < 0 || L < 0) return fail(SSM_ERR_INVALID_ARGUMENT, "B and L must be >= 0");
  if (H < 1) return fail(SSM_ERR_INVALID_ARGUMENT, "H=%lld must be >= 1", (long long)H);
  if (G < 1 || H % G != 0)
    return fail(SSM_ERR_INVALID_ARGUMENT, "G=%lld must be >= 1 and divide H=%lld", (long long)G, (long long)H);
  if (!valid_dtype(io)) return fail(SSM_ERR_INVALID_ARGUMENT, "unknown io_dtype %d", (int)io);
  if (io != SSM_BF16) return fail(SSM_ERR_UNSUPPORTED, "ssd_chunk_bwd supports io_dtype SSM_BF16 only");
  if (P != 64) return fail(SSM_ERR_UNSUPPORTED, "P=%lld: supported head dim is 64", (long long)P);
  if (N != 64 && N != 128) return fail(SSM_ERR_UNSUPPORTED, "N=%lld: supported 64, 128", (long long)N);
  const int64_t Q = ssm::kSsdBwdQ;
  if ((L + Q - 1) / Q > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "L=%lld: at most 65535 chunks of %lld tokens", (long long)L, (long long)Q);
  if (B * G > 65535 || H > 65535)
    return fail(SSM_ERR_UNSUPPORTED, "B*G=%lld and H=%lld must each be <= 65535", (long long)(B * G), (long long)H);
  if (!A || !dA) return fail(SSM_ERR_INVALID_ARGUMENT, "A and dA must not be NULL");
  if (z && !dz) return fail(SSM_ERR_INVALID_ARGUMENT, "dz must be given with z");
  const bool dpc = dskip_per_channel != 0;
  const size_t tok = (size_t)(B * L * H * P) * 2, th = (size_t)(B * L * H) * 2;
  const size_t bc = (size_t)(B * L * G * N) * 2, bcg = (size_t)(B * L * G * N) * 4;
  const size_t stb = (size_t)(B * H * P * N) * 4, vh = (size_t)H * 4;
  const size_t vd = (size_t)(dpc ? H * P : H) * 4;
  if (B > 0 && L > 0) {
    if (!x || !delta || !Bm || !Cm || !dy || !dx || !ddelta || !dBm || !dCm)
      return fail(SSM_ERR_INVALID_ARGUMENT, "x, delta, Bm, Cm, dy, dx, ddelta, dBm and dCm must not be NULL");
    if (!aligned16(x) || !aligned16(Bm) || !aligned16(Cm) || !aligned16(dy) || !aligned16(dx) ||
        !aligned16(dBm) || !aligned16(dCm) || (z && !aligned16(z)) || (dz && !aligned16(dz)) ||
        (Dskip && dpc && !aligned16(Dskip)))
      return fail(SSM_ERR_INVALID_ARGUMENT, "per-token tensors must be 16-byte aligned");
  }
  const void* ins[] = {x, delta, z, Bm, Cm, dy, A, delta_bias, Dskip, h0, dh_last};
  const size_t insz[] = {tok, th, tok, bc, bc, tok, vh, vh, vd, stb, stb};
  void* outs[] = {dx, ddelta, z ? dz : nullptr, dA, dBm, dCm, dDskip, ddelta_bias, dh0};
  const size_t outsz[] = {tok, th, tok, vh, bcg, bcg, vd, vh, stb};
  for (int o = 0; o < 9; ++o) {
    for (int k = 0; k < 11; ++k)
      if (overlaps(outs[o], outsz[o], ins[k], insz[k]))
        return fail(SSM_ERR_INVALID_ARGUMENT, "a gradient output overlaps an input");
    for (int k = o + 1; k < 9; ++k)
      if (overlaps(outs[o], outsz[o], outs[k], outsz[k]))
        return fail(SSM_ERR_INVALID_ARGUMENT, "two gradient outputs overlap");
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (B == 0 || L == 0) {
    // empty sums: parameter gradients are zero; dh0 is dh_last passed through (or zero)
    hipError_t e = hipMemsetAsync(dA, 0, vh, st);
    if (e == hipSuccess && dDskip) e = hipMemsetAsync(dDskip, 0, vd, st);
    if (e == hipSuccess && ddelta_bias) e = hipMemsetAsync(ddelta_bias, 0, vh, st);
    if (e == hipSuccess && dh0 && B > 0)
      e = dh_last ? hipMemcpyAsync(dh0, dh_last, stb, hipMemcpyDeviceToDevice, st) : hipMemsetAsync(dh0, 0, stb, st);
    return from_hip(e, "empty backward");
  }
  const int64_t hb = ssd_bwd_heads_per_wg(B, L, H, G);
  const size_t need = ssm::ssd_bwd_workspace_bytes(B, L, H, P, N, G, hb);
  if (!ws) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace is NULL; %zu bytes needed", need);
  if (ws_bytes < need) return fail(SSM_ERR_WORKSPACE_TOO_SMALL, "workspace %zu bytes < %zu needed", ws_bytes, need);
  if (!aligned16(ws)) return fail(SSM_ERR_INVALID_ARGUMENT, "workspace must be 16-byte aligned");
  ssm::SsdBwdParams bp{};
  ssm::SsdParams& p = bp.f;
  p.B = B; p.L = L; p.H = H; p.P = P; p.N = N; p.Q = Q; p.G = G;
  p.x = x; p.delta = delta; p.z = z; p.Bm = Bm; p.Cm = Cm;
  p.delta_bias = delta_bias; p.A = A; p.Dskip = Dskip; p.h0 = h0;
  p.dskip_per_channel = Dskip && dpc ? 1 : 0;
  p.delta_softplus = delta_softplus ? 1 : 0;
  p.h_last = nullptr;
  p.dy = dy; p.dh_last = dh_last; p.dh0 = dh0;
  bp.dx = dx; bp.ddelta = ddelta; bp.dz = z ? dz : nullptr; bp.dA = dA; bp.dBm = dBm; bp.dCm = dCm;
  bp.dDskip = dDskip; bp.ddelta_bias = ddelta_bias; bp.hb = hb;
  ssm::ssd_bwd_workspace_carve(bp, ws);
  return from_hip(ssm::launch_ssd_bwd(bp, st), "ssd_chunk_bwd launch");
}

}  // extern "C"
