/*
 * lsec_floor.h -- measurement aids of liblsec.so (gfx950). They are not
 * operations of the LSE-weighted combine: they give the reference points
 * that the library's kernels are timed against on the same device, in the
 * same process and cache state:
 *  - lsec_floor_empty : a launch that does no work (one 64-lane wave), i.e.
 *                       the duration no kernel launch can go below;
 *  - lsec_floor_read  : a plain streaming read of a buffer with the same
 *                       16-byte non-temporal loads the combine uses, i.e. the
 *                       rate the device reaches for those bytes with no
 *                       arithmetic, no layout and (almost) no writes;
 *  - lsec_floor_copy  : a plain copy with those loads and 16-byte
 *                       non-temporal stores, the same for calls that write as
 *                       much as they read (pack, unpack, corrected partial);
 *  - lsec_time_next_launch : times the next kernel the library launches from
 *                       the calling thread by its own dispatch, so that a
 *                       caller can time single short launches without the
 *                       cost of separate event markers around them.
 * A combining call that moves b bytes cannot finish faster than a plain read
 * of b bytes, a call that reads and writes b / 2 bytes each not faster than
 * a plain copy of b / 2 bytes, and no call faster than an empty launch; for
 * calls of a few tens of MB these are close to each other.
 *
 * Conventions are those of lsec.h: device pointers, the caller allocates,
 * work is enqueued on `stream` (NULL = the null stream), arguments are checked
 * before anything is enqueued and a status code of lsec.h is returned.
 */
#ifndef LSEC_FLOOR_H
#define LSEC_FLOOR_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * lsec_time_next_launch -- arm a pair of events for the next kernel that this
 * library launches from the calling thread (any entry point of lsec.h or of
 * this header; each launches exactly one kernel). That launch records its
 * kernel's start in `start` and its end in `stop`, taken from the kernel's own
 * dispatch (hipExtLaunchKernelGGL), so hipEventElapsedTime(start, stop) is
 * the kernel's duration without the time of event markers recorded around
 * it; the pair is then disarmed. Later launches are plain launches again.
 *   start, stop : hipEvent_t handles the caller created (hipEventCreate) on
 *                 the device of the next launch; both NULL disarms a pair
 *                 that no launch has taken yet (a call that fails its
 *                 argument checks launches nothing and leaves it armed)
 * Not for calls under stream capture. Arming is per thread: a launch from
 * another thread is never timed by it.
 * Errors: NULL (exactly one of the two is NULL).
 */
int lsec_time_next_launch(void* start, void* stop);

/*
 * lsec_floor_empty -- launch one wave of 64 lanes that returns at once.
 * Errors: LAUNCH.
 */
int lsec_floor_empty(void* stream);

/*
 * lsec_floor_read_blocks -- number of 32-bit words `sink` must hold for
 * lsec_floor_read of `bytes` bytes (one per 16 KiB of input, rounded up);
 * -1 if bytes is negative or not a multiple of 16.
 */
int64_t lsec_floor_read_blocks(int64_t bytes);

/*
 * lsec_floor_read -- read `bytes` bytes of `src` once.
 *   src   : bytes / 16 chunks of 16 bytes, 16-byte aligned (device memory)
 *   bytes : >= 0, a multiple of 16
 *   sink  : lsec_floor_read_blocks(bytes) uint32 words (written): word k is
 *           the XOR of the 32-bit words of src's k-th 16 KiB (the last one
 *           may be shorter), so the XOR of all of sink is the XOR of all of
 *           src -- the reads cannot be optimised away, and a test can check
 *           that every byte was read.
 * A lane keeps four 16-byte loads in flight; a 256-lane block reads one
 * contiguous 16 KiB run and stores one word.
 * Errors: SHAPE (bytes negative or not a multiple of 16), NULL, ALIGNMENT
 * (src not 16-byte aligned, sink not 4-byte aligned), LAUNCH.
 */
int lsec_floor_read(const void* src, int64_t bytes, uint32_t* sink, void* stream);

/*
 * lsec_floor_copy -- copy `bytes` bytes from `src` to `dst` once.
 *   src, dst : bytes / 16 chunks of 16 bytes each, 16-byte aligned (device
 *              memory); the two must not overlap
 *   bytes    : >= 0, a multiple of 16
 * A lane keeps four 16-byte loads in flight, then stores them; a 256-lane
 * block copies one contiguous 16 KiB run.
 * Errors: SHAPE (bytes negative or not a multiple of 16), NULL, ALIGNMENT
 * (src or dst not 16-byte aligned), LAUNCH.
 */
int lsec_floor_copy(const void* src, void* dst, int64_t bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LSEC_FLOOR_H */
