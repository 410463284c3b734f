// Dispatch over the 34 valid (l_in, l_sh, l_out) triples with l <= 3 (internal).
#pragma once

#define ETPC_TRIPLE_DISPATCH(LI_, LS_, LO_, CALL)          \
  switch ((LI_) * 16 + (LS_) * 4 + (LO_)) {                \
    case 0: return CALL(0, 0, 0);          \
    case 5: return CALL(0, 1, 1);          \
    case 10: return CALL(0, 2, 2);          \
    case 15: return CALL(0, 3, 3);          \
    case 17: return CALL(1, 0, 1);          \
    case 20: return CALL(1, 1, 0);          \
    case 21: return CALL(1, 1, 1);          \
    case 22: return CALL(1, 1, 2);          \
    case 25: return CALL(1, 2, 1);          \
    case 26: return CALL(1, 2, 2);          \
    case 27: return CALL(1, 2, 3);          \
    case 30: return CALL(1, 3, 2);          \
    case 31: return CALL(1, 3, 3);          \
    case 34: return CALL(2, 0, 2);          \
    case 37: return CALL(2, 1, 1);          \
    case 38: return CALL(2, 1, 2);          \
    case 39: return CALL(2, 1, 3);          \
    case 40: return CALL(2, 2, 0);          \
    case 41: return CALL(2, 2, 1);          \
    case 42: return CALL(2, 2, 2);          \
    case 43: return CALL(2, 2, 3);          \
    case 45: return CALL(2, 3, 1);          \
    case 46: return CALL(2, 3, 2);          \
    case 47: return CALL(2, 3, 3);          \
    case 51: return CALL(3, 0, 3);          \
    case 54: return CALL(3, 1, 2);          \
    case 55: return CALL(3, 1, 3);          \
    case 57: return CALL(3, 2, 1);          \
    case 58: return CALL(3, 2, 2);          \
    case 59: return CALL(3, 2, 3);          \
    case 60: return CALL(3, 3, 0);          \
    case 61: return CALL(3, 3, 1);          \
    case 62: return CALL(3, 3, 2);          \
    case 63: return CALL(3, 3, 3);          \
    default: return hipErrorInvalidValue;                 \
  }
