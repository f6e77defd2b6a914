"""Counter-based random numbers, bit-identical on the host (numpy) and the device.

Definition (SplitMix64, Steele, Lea and Flood, "Fast splittable pseudorandom
number generators", OOPSLA 2014; constants as published by S. Vigna):

    mix64(z):  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9
               z = (z ^ (z >> 27)) * 0x94D049BB133111EB
               return z ^ (z >> 31)                      (all mod 2^64)

    key(seed, tid) = mix64(seed * 0x9E3779B97F4A7C15 + tid * 0xD1B54A32D192ED03)
    u64(seed, tid, n) = mix64(key(seed, tid) + (n + 1) * 0x9E3779B97F4A7C15)

Element ``n`` of tensor ``tid`` therefore depends only on (seed, tid, n), so any
slice of a tensor that lives only in device memory can be regenerated on the
host.

Normal variates use the Irwin-Hall construction: the four 16-bit fields of
u64 are summed (an integer in [0, 262140]), centred, and multiplied by the
float32 constant 1/sd with sd = sqrt((65536**2 - 1) / 3). Both steps are exact
or correctly rounded in IEEE fp32, so host and device produce the same bits.
The variates are bounded by +-3.46 and have mean 0 and variance 1.

bf16 values are produced from fp32 by round-to-nearest-even on the bit
pattern and are stored as uint16.
"""
import numpy as np

_GOLDEN = np.uint64(0x9E3779B97F4A7C15)
_TIDMUL = np.uint64(0xD1B54A32D192ED03)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
IH_CENTER = 131070
IH_INV_SD = np.float32(1.0 / np.sqrt((65536.0 ** 2 - 1.0) / 3.0))

# Tensor identifiers: one stream per role.
TENSOR_IDS = {
    "q": 1, "k": 2, "v": 3, "lmk": 4, "lmk_noise": 5, "bias": 6, "dout": 7,
    "needle_u": 8, "needle_pos": 9, "resid": 10, "lq": 11, "dlmk": 12, "dbias": 13,
    "qret_a": 14, "qret_b": 15, "ties": 16,
}


def _mix64(z):
    with np.errstate(over="ignore"):
        z = (z ^ (z >> np.uint64(30))) * _M1
        z = (z ^ (z >> np.uint64(27))) * _M2
    return z ^ (z >> np.uint64(31))


def splitmix64_key(seed, tid):
    with np.errstate(over="ignore"):
        z = np.uint64(seed) * _GOLDEN + np.uint64(tid) * _TIDMUL
    return _mix64(np.asarray(z, dtype=np.uint64))


def uniform_u64(seed, tid, idx):
    """Raw 64-bit draws for element indices ``idx`` (any integer array)."""
    key = splitmix64_key(seed, tid)
    n = np.asarray(idx, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = key + (n + np.uint64(1)) * _GOLDEN
    return _mix64(z)


def normal_f32(seed, tid, idx, scale=1.0):
    """Approximately N(0, scale^2) float32 values for element indices ``idx``."""
    u = uniform_u64(seed, tid, idx)
    m = np.uint64(0xFFFF)
    s = ((u & m) + ((u >> np.uint64(16)) & m) + ((u >> np.uint64(32)) & m)
         + ((u >> np.uint64(48)) & m)).astype(np.int64) - IH_CENTER
    x = s.astype(np.float32) * IH_INV_SD
    if scale != 1.0:
        x = x * np.float32(scale)
    return x


def f32_to_bf16_bits(x):
    """Round float32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b):
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16_bits(seed, tid, idx, scale=1.0):
    return f32_to_bf16_bits(normal_f32(seed, tid, idx, scale))
