// Decode-ahead scheduling of "hard" matrices ("Unweight: how we compressed an
// LLM 22% without sacrificing quality": the paragraph on hard and easy layers,
// the figure caption on decoding in separate streams during initial load,
// attention and easy MLPs, and the paragraph on splitting the compute units
// between decode and matmul).
//
// A scheduler owns a side stream and a ring of decode slots (caller-owned
// device memory).  uw_sched_prefetch records a fork event on the caller's
// stream, makes the side stream wait for it, decompresses the matrix into a
// free slot there and records the slot's ready event; uw_sched_gemm makes the
// caller's stream wait for that event and multiplies from the slot.  The
// decode therefore overlaps whatever the caller enqueues between the two
// calls (the easy projections), and every dependency is an event recorded
// inside the call sequence, so the sequence can be captured in a HIP graph.
// A slot is free again once its product has been enqueued: the next decode
// into it waits (through its fork event) for everything the caller's stream
// held at that point, the product included.
//
// The side stream may be limited to a subset of the compute units
// (hipExtStreamCreateWithCUMask): CU i is taken when i % 32 < k * 32 / n for
// n CUs and k asked, which gives every XCD the same share whether the CU
// numbering interleaves the XCDs or blocks them.
#include <hip/hip_runtime.h>  // hipExtStreamCreateWithCUMask is declared in its runtime API

#include <cstring>
#include <string>
#include <vector>

#include "uw_internal.h"

struct uw_sched {
  int device = 0;
  hipStream_t side = nullptr;
  uint8_t* slots = nullptr;
  size_t slot_bytes = 0;
  int n_slots = 0;
  int decode_cus = 0;
  std::vector<hipEvent_t> fork, ready;
  std::vector<const uw_matrix*> held;  // the matrix a slot holds until its product is enqueued
  int next = 0;
};

using namespace uw;

namespace {

void destroy_events(uw_sched* s) {
  for (hipEvent_t e : s->fork)
    if (e) (void)hipEventDestroy(e);
  for (hipEvent_t e : s->ready)
    if (e) (void)hipEventDestroy(e);
  s->fork.clear();
  s->ready.clear();
}

}  // namespace

extern "C" {

int uw_sched_create(void* d_slots, size_t slot_bytes, int n_slots, int decode_cus, uw_sched** out) {
  if (!d_slots || !out || n_slots < 1 || n_slots > 64 || slot_bytes < 256)
    return fail(UW_ERR_INVALID, "uw_sched_create: slots, 1..64 of them, and an output pointer are needed");
  if (reinterpret_cast<uintptr_t>(d_slots) % 256 || slot_bytes % 256)
    return fail(UW_ERR_INVALID, "uw_sched_create: slots must be 256-byte aligned and a multiple of 256 bytes");
  int dev = -1, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return fail(UW_ERR_HIP, "uw_sched_create: no current HIP device");
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    return fail(UW_ERR_HIP, "uw_sched_create: cannot read the compute unit count");
  if (decode_cus < 0 || decode_cus > cus) return fail(UW_ERR_INVALID, "uw_sched_create: decode_cus out of range");
  uw_sched* s = new uw_sched();
  s->device = dev;
  s->slots = static_cast<uint8_t*>(d_slots);
  s->slot_bytes = slot_bytes;
  s->n_slots = n_slots;
  s->decode_cus = decode_cus;
  hipError_t e;
  if (decode_cus == 0 || decode_cus == cus) {
    e = hipStreamCreateWithFlags(&s->side, hipStreamNonBlocking);
  } else {
    std::vector<uint32_t> mask((cus + 31) / 32, 0u);
    const int per32 = std::max(1, decode_cus * 32 / cus);
    int taken = 0;
    for (int i = 0; i < cus && taken < decode_cus; ++i)
      if (i % 32 < per32) {
        mask[i / 32] |= 1u << (i % 32);
        ++taken;
      }
    s->decode_cus = taken;
    e = hipExtStreamCreateWithCUMask(&s->side, uint32_t(mask.size()), mask.data());
  }
  if (e != hipSuccess) {
    delete s;
    return fail(UW_ERR_HIP, std::string("uw_sched_create: stream: ") + hipGetErrorString(e));
  }
  s->fork.assign(n_slots, nullptr);
  s->ready.assign(n_slots, nullptr);
  s->held.assign(n_slots, nullptr);
  for (int i = 0; i < n_slots; ++i) {
    if (hipEventCreateWithFlags(&s->fork[i], hipEventDisableTiming) != hipSuccess ||
        hipEventCreateWithFlags(&s->ready[i], hipEventDisableTiming) != hipSuccess) {
      destroy_events(s);
      (void)hipStreamDestroy(s->side);
      delete s;
      return fail(UW_ERR_HIP, "uw_sched_create: events");
    }
  }
  *out = s;
  return UW_OK;
}

void uw_sched_destroy(uw_sched* s) {
  if (!s) return;
  (void)hipStreamSynchronize(s->side);
  destroy_events(s);
  (void)hipStreamDestroy(s->side);
  delete s;
}

int uw_sched_decode_cus(const uw_sched* s) { return s ? s->decode_cus : -1; }

int uw_sched_prefetch(uw_sched* s, const uw_matrix* m, void* stream, int* slot) {
  if (!s || !m || !slot) return fail(UW_ERR_INVALID, "uw_sched_prefetch: null pointer");
  if (m->device != s->device) return fail(UW_ERR_INVALID, "uw_sched_prefetch: matrix and scheduler on different devices");
  if (size_t(m->h.rows) * size_t(m->h.cols) * 2 > s->slot_bytes)
    return fail(UW_ERR_NOSPACE, "uw_sched_prefetch: the decompressed matrix does not fit in a slot");
  int k = -1;
  for (int i = 0; i < s->n_slots; ++i) {
    const int j = (s->next + i) % s->n_slots;
    if (!s->held[j]) {
      k = j;
      break;
    }
  }
  if (k < 0) return fail(UW_ERR_NOSPACE, "uw_sched_prefetch: every slot holds a matrix whose product is not enqueued");
  hipStream_t caller = static_cast<hipStream_t>(stream);
  // a side stream limited to part of the compute units is not joined into a
  // graph capture: one such captured sequence left the process unable to
  // release the stream, so the combination is refused
  if (s->decode_cus > 0) {
    hipStreamCaptureStatus st = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(caller, &st) != hipSuccess) return fail(UW_ERR_HIP, "uw_sched_prefetch: capture status");
    if (st != hipStreamCaptureStatusNone)
      return fail(UW_ERR_UNSUPPORTED,
                  "uw_sched_prefetch: a scheduler with a compute-unit mask cannot be used under graph capture");
  }
  // the decode starts once the caller's stream has reached this point (the
  // slot's previous product, enqueued before, has then completed)
  if (hipEventRecord(s->fork[k], caller) != hipSuccess || hipStreamWaitEvent(s->side, s->fork[k], 0) != hipSuccess)
    return fail(UW_ERR_HIP, "uw_sched_prefetch: fork event");
  uint16_t* dst = reinterpret_cast<uint16_t*>(s->slots + size_t(k) * s->slot_bytes);
  if (int rc = launch_decompress(m, dst, m->h.cols, s->side)) return rc;
  if (hipEventRecord(s->ready[k], s->side) != hipSuccess) return fail(UW_ERR_HIP, "uw_sched_prefetch: ready event");
  s->held[k] = m;
  s->next = (k + 1) % s->n_slots;
  *slot = k;
  return UW_OK;
}

int uw_sched_gemm(uw_sched* s, int slot, const void* d_X, int64_t batch, int64_t ldx, int xt, void* d_Y, int64_t ldy,
                  int yt, void* stream) {
  if (!s || slot < 0 || slot >= s->n_slots) return fail(UW_ERR_INVALID, "uw_sched_gemm: bad scheduler or slot");
  const uw_matrix* m = s->held[slot];
  if (!m) return fail(UW_ERR_INVALID, "uw_sched_gemm: the slot holds no prefetched matrix");
  const int64_t rows = m->h.rows, cols = m->h.cols;
  if (batch < 1 || !d_X || !d_Y || (xt != UW_F32 && xt != UW_BF16) || (yt != UW_F32 && yt != UW_BF16) || ldx < cols ||
      (batch > 1 && ldy < rows))
    return fail(UW_ERR_INVALID, "uw_sched_gemm: bad operands");
  std::string why;
  if (!bf16_gemm_supported(cols, batch, xt, &why)) return fail(UW_ERR_UNSUPPORTED, "uw_sched_gemm: " + why);
  hipStream_t caller = static_cast<hipStream_t>(stream);
  if (hipStreamWaitEvent(caller, s->ready[slot], 0) != hipSuccess) return fail(UW_ERR_HIP, "uw_sched_gemm: join event");
  const uint16_t* W = reinterpret_cast<const uint16_t*>(s->slots + size_t(slot) * s->slot_bytes);
  const int rc = launch_bf16_gemm(W, rows, cols, cols, d_X, batch, ldx, xt, d_Y, ldy, yt, stream);
  s->held[slot] = nullptr;  // enqueued: the next decode into this slot waits for it through its fork event
  return rc;
}

}  // extern "C"
